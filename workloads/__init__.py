"""Seeded synthetic inputs for paged MLA decode.

This module is shared by the CPU oracle's tests, the GPU parity tests and the
benchmark. It only draws random numbers and stores them in the formats the
decode consumes (bf16 bit patterns, OCP e4m3fn codes with a per-tensor scale,
int32 CSR index lists). It holds none of the attention arithmetic.

Workload shapes follow the pages' serving cases: the 7+1 token speculative
verify pass (ATOM pull request 2760, "Validation"), the batch-8, block-8,
8k-context non-causal draft block (vLLM pull request 53001, "Purpose") and
the 128-head fp8 decode of the persistent-kernel gate (ATOM pull request
2462, "Summary", part 2). Real model weights and datasets are not needed:
every value is N(0, 1).

Recipe (per config k): ``rng = numpy.random.default_rng(seed)``; draw, in
this order, the KV lengths, a permutation of the pool's slots (row i takes
the next L_i slots, so rows are disjoint), the pool values (every slot), then
Q. bf16 storage is round-to-nearest-even from float32; fp8 storage uses a
per-tensor scale amax/448, values divided by it, clamped to +-448 and
rounded to nearest even.
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional, Sequence

import numpy as np

D_LATENT = 576   # 512 compressed ("nope") dims + 64 RoPE dims per KV slot
D_V = 512        # V is the first 512 dims of the latent row
SM_SCALE = np.float32(1.0 / math.sqrt(192.0))

BF16 = "bf16"
FP8 = "fp8"


@dataclasses.dataclass
class Case:
    """One decode batch in stored form (host numpy arrays)."""
    name: str
    rows: int
    q_len: int              # q_len_max; qo_indptr may be ragged below it
    heads: int
    causal: bool
    q_dtype: str
    kv_dtype: str
    q_codes: np.ndarray     # uint16 (bf16 bits) or uint8 (e4m3fn) [T, H, 576]
    q_scale: Optional[float]    # float32 value, None for bf16 (scale 1)
    pool_codes: np.ndarray  # uint16 or uint8 [P, 576]
    kv_scale: Optional[float]
    qo_indptr: np.ndarray   # int32 [rows+1]
    kv_indptr: np.ndarray   # int32 [rows+1]
    kv_indices: np.ndarray  # int32 [nnz]
    sm_scale: np.float32
    # extra disjoint index lists over the same pool (benchmark rotation)
    alt_kv_indices: List[np.ndarray] = dataclasses.field(default_factory=list)

    @property
    def kv_lens(self) -> np.ndarray:
        return np.diff(self.kv_indptr).astype(np.int32)

    @property
    def q_lens(self) -> np.ndarray:
        return np.diff(self.qo_indptr).astype(np.int32)

    @property
    def num_tokens(self) -> int:
        return int(self.qo_indptr[-1])

    @property
    def num_slots(self) -> int:
        return int(self.pool_codes.shape[0])


def _to_bf16_bits(x: np.ndarray) -> np.ndarray:
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _to_fp8(x: np.ndarray):
    """Per-tensor scale amax/448, clamp to +-448, RNE cast to e4m3fn.

    torch's cast does not saturate (an out-of-range value becomes NaN), so the
    clamp comes first. Returns (codes uint8, scale as a Python float holding a
    float32 value)."""
    import torch
    x = np.ascontiguousarray(x, dtype=np.float32)
    amax = float(np.abs(x).max()) if x.size else 0.0
    scale = np.float32(amax / 448.0) if amax > 0 else np.float32(1.0)
    y = x / scale
    np.clip(y, -448.0, 448.0, out=y)
    codes = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return codes, float(scale)


def _store(x: np.ndarray, dtype: str):
    if dtype == BF16:
        return _to_bf16_bits(x), None
    if dtype == FP8:
        return _to_fp8(x)
    raise ValueError(dtype)


def make_case(seed: int, kv_lens: Sequence[int] | None, heads: int, q_len: int,
              q_dtype: str, kv_dtype: str, causal: bool, pool_slots: int,
              name: str = "case", lens_fn=None, q_lens: Sequence[int] | None = None,
              kv_indptr_offset: int = 0, extra_index_sets: int = 0,
              shared_slots: bool = False) -> Case:
    """General seeded generator.

    ``lens_fn(rng)`` draws the lengths when ``kv_lens`` is None (so the draw
    happens first, as the recipe says). ``q_lens`` gives a ragged query block
    per row (default: q_len for every row). ``kv_indptr_offset`` shifts the
    whole CSR so that kv_indptr[0] != 0 (an offset list; the leading entries of
    kv_indices are then unused padding). ``shared_slots`` makes every row read
    the same slots (identical rows when Q rows are also equal)."""
    rng = np.random.default_rng(seed)
    lens = np.asarray(lens_fn(rng) if kv_lens is None else kv_lens, dtype=np.int64)
    rows = int(lens.shape[0])
    total = int(lens.sum())
    perm = rng.permutation(pool_slots).astype(np.int64)
    need = (1 + extra_index_sets) * (int(lens.max()) if shared_slots and rows else total)
    if need > pool_slots:
        raise ValueError(f"pool of {pool_slots} slots cannot hold {need} disjoint keys")
    pool = rng.standard_normal((pool_slots, D_LATENT), dtype=np.float32)
    pool_codes, kv_scale = _store(pool, kv_dtype)
    del pool
    ql = np.full(rows, q_len, dtype=np.int64) if q_lens is None else np.asarray(q_lens, np.int64)
    if ql.shape[0] != rows or (ql > q_len).any() or (ql < 0).any():
        raise ValueError("q_lens must have one entry per row, each in [0, q_len]")
    T = int(ql.sum())
    q = rng.standard_normal((T, heads, D_LATENT), dtype=np.float32)
    q_codes, q_scale = _store(q, q_dtype)
    del q

    qo_indptr = np.zeros(rows + 1, dtype=np.int32)
    qo_indptr[1:] = np.cumsum(ql)
    kv_indptr = np.zeros(rows + 1, dtype=np.int32)
    kv_indptr[1:] = np.cumsum(lens)
    kv_indptr += kv_indptr_offset

    def index_set(k):
        if shared_slots:
            base = perm[k * int(lens.max()):(k + 1) * int(lens.max())]
            flat = np.concatenate([base[:n] for n in lens]) if rows else base[:0]
        else:
            flat = perm[k * total:(k + 1) * total]
        pad = rng.integers(0, pool_slots, kv_indptr_offset) if kv_indptr_offset else np.zeros(0, np.int64)
        return np.concatenate([pad, flat]).astype(np.int32)

    kv_indices = index_set(0)
    alts = [index_set(k) for k in range(1, extra_index_sets + 1)]
    return Case(name=name, rows=rows, q_len=q_len, heads=heads, causal=causal,
                q_dtype=q_dtype, kv_dtype=kv_dtype, q_codes=q_codes, q_scale=q_scale,
                pool_codes=pool_codes, kv_scale=kv_scale, qo_indptr=qo_indptr,
                kv_indptr=kv_indptr, kv_indices=kv_indices, sm_scale=SM_SCALE,
                alt_kv_indices=alts)


def make_sparse_case(seed: int, rows: int, ctx: Sequence[int], window: int, topk: int, heads: int,
                     q_len: int, q_dtype: str, kv_dtype: str, name: str = "sparse",
                     extra_index_sets: int = 0) -> Case:
    """Sparse (top-k) index lists over a row-dense pool: row b owns C_b
    consecutive slots (its context, C_b drawn uniformly in [ctx[0], ctx[1]]);
    its list is `topk` positions drawn without replacement from the first
    C_b - window positions, ascending, followed by the last `window` positions
    (a sliding window plus selected tokens, the DeepSeek-V4 CSA list of ATOM
    pull request 2462, Summary part 1). Non-causal. Only listed slots get
    values (the rest of the pool is zero and never read). Extra index sets
    redraw the top-k part (benchmark rotation).

    Draw order: contexts, top-k positions per row (and per extra set), values
    of the listed slots, then Q."""
    rng = np.random.default_rng(seed)
    C = rng.integers(int(ctx[0]), int(ctx[1]) + 1, rows).astype(np.int64)
    base = np.concatenate([[0], np.cumsum(C)[:-1]]).astype(np.int64)
    pool_slots = int(C.sum())

    def draw_lists():
        out = []
        for b in range(rows):
            pre = int(C[b]) - window
            sel = np.sort(rng.choice(pre, size=min(topk, pre), replace=False)) if pre > 0 else np.zeros(0, np.int64)
            win = np.arange(max(pre, 0), int(C[b]), dtype=np.int64)
            out.append(base[b] + np.concatenate([sel, win]))
        return out

    sets = [draw_lists() for _ in range(1 + extra_index_sets)]
    lens = np.array([len(x) for x in sets[0]], dtype=np.int64)
    used = np.unique(np.concatenate([np.concatenate(s) for s in sets]))
    vals = rng.standard_normal((used.shape[0], D_LATENT), dtype=np.float32)
    codes, kv_scale = _store(vals, kv_dtype)
    del vals
    pool_codes = np.zeros((pool_slots, D_LATENT), dtype=codes.dtype)
    pool_codes[used] = codes
    T = rows * q_len
    q = rng.standard_normal((T, heads, D_LATENT), dtype=np.float32)
    q_codes, q_scale = _store(q, q_dtype)
    del q
    qo_indptr = (np.arange(rows + 1) * q_len).astype(np.int32)
    kv_indptr = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    flat = [np.concatenate(s).astype(np.int32) for s in sets]
    return Case(name=name, rows=rows, q_len=q_len, heads=heads, causal=False, q_dtype=q_dtype,
                kv_dtype=kv_dtype, q_codes=q_codes, q_scale=q_scale, pool_codes=pool_codes,
                kv_scale=kv_scale, qo_indptr=qo_indptr, kv_indptr=kv_indptr, kv_indices=flat[0],
                sm_scale=SM_SCALE, alt_kv_indices=flat[1:])


# The workloads. Each entry: (seed, lens or lens_fn, heads, q_len, q_dtype,
# kv_dtype, causal, pool slots); "sparse" entries use make_sparse_case.
def _lens_c2(rng):
    return rng.integers(1024, 8193, 32)


def _lens_c5(rng):
    x = np.exp(rng.normal(math.log(2048.0), 1.0, 256))
    return np.clip(np.rint(x), 16, 16384).astype(np.int64)


CONFIGS = {
    # 2 rows, q_len 1, 16 heads, bf16, lengths 37 and 128, 4096-slot pool, causal
    "tiny_causal": dict(seed=1, kv_lens=[37, 128], heads=16, q_len=1, q_dtype=BF16,
                        kv_dtype=BF16, causal=True, pool_slots=4096),
    # 32 rows, 7 draft + 1 token verify, 128 heads, bf16, lengths U[1024, 8192], 512k pool
    "verify_causal": dict(seed=2, lens_fn=_lens_c2, heads=128, q_len=8, q_dtype=BF16,
                          kv_dtype=BF16, causal=True, pool_slots=524288),
    # the same batch (same seed, so the same lengths) with an fp8 e4m3 KV cache
    # and bf16 Q: the shape the headline metric names (128 heads, q_len 8, fp8 KV)
    "verify_causal_fp8kv": dict(seed=2, lens_fn=_lens_c2, heads=128, q_len=8, q_dtype=BF16,
                                kv_dtype=FP8, causal=True, pool_slots=524288),
    # 8 rows, block of 8, 64 heads, fp8 Q and KV, 8192 keys per row, non-causal
    "draft_noncausal": dict(seed=3, kv_lens=[8192] * 8, heads=64, q_len=8, q_dtype=FP8,
                            kv_dtype=FP8, causal=False, pool_slots=524288),
    # 4 rows, q_len 1, 128 heads, bf16 Q, fp8 KV, 32k..128k keys, uniform split plan
    "longctx_split": dict(seed=4, kv_lens=[32768, 65536, 98304, 131072], heads=128, q_len=1,
                          q_dtype=BF16, kv_dtype=FP8, causal=True, pool_slots=524288),
    # 256 rows, q_len 2, 128 heads, bf16 Q, fp8 KV, lognormal lengths, per-call plan
    "ragged_persistent_causal": dict(seed=5, lens_fn=_lens_c5, heads=128, q_len=2, q_dtype=BF16,
                                     kv_dtype=FP8, causal=True, pool_slots=1048576),
    "ragged_persistent_noncausal": dict(seed=5, lens_fn=_lens_c5, heads=128, q_len=2, q_dtype=BF16,
                                        kv_dtype=FP8, causal=False, pool_slots=1048576),
    # 64 rows, q_len 2, 128 heads, bf16 Q, fp8 KV: top-k 2048 + window 128 of
    # 8k..32k-token contexts (sparse index lists, non-causal)
    "sparse_topk": dict(seed=6, sparse=dict(rows=64, ctx=(8192, 32768), window=128, topk=2048),
                        heads=128, q_len=2, q_dtype=BF16, kv_dtype=FP8, causal=False, pool_slots=None),
}


def make_config(name: str, extra_index_sets: int = 0) -> Case:
    spec = dict(CONFIGS[name])
    seed = spec.pop("seed")
    if "sparse" in spec:
        sp = spec["sparse"]
        return make_sparse_case(seed, sp["rows"], sp["ctx"], sp["window"], sp["topk"], spec["heads"],
                                spec["q_len"], spec["q_dtype"], spec["kv_dtype"], name=name,
                                extra_index_sets=extra_index_sets)
    lens = spec.pop("kv_lens", None)
    return make_case(seed, lens, name=name, extra_index_sets=extra_index_sets, **spec)


def config_lengths(name: str) -> np.ndarray:
    """The config's KV lengths without generating the pool (same draw)."""
    spec = CONFIGS[name]
    if "sparse" in spec:
        sp = spec["sparse"]
        C = np.random.default_rng(spec["seed"]).integers(sp["ctx"][0], sp["ctx"][1] + 1, sp["rows"])
        return np.array([min(sp["topk"], max(int(c) - sp["window"], 0)) + min(sp["window"], int(c))
                         for c in C], dtype=np.int64)
    if "kv_lens" in spec:
        return np.asarray(spec["kv_lens"], dtype=np.int64)
    return np.asarray(spec["lens_fn"](np.random.default_rng(spec["seed"])), dtype=np.int64)


def index_set_capacity(name: str) -> int:
    """How many index lists (the first plus alternates) the config can draw
    for benchmark rotation: disjoint lists for the dense configs, redrawn
    top-k lists for the sparse one."""
    spec = CONFIGS[name]
    if "sparse" in spec:
        return 3
    return max(1, int(spec["pool_slots"] // max(int(config_lengths(name).sum()), 1)))


def make_logit_jump_case(seed: int, kv_lens: Sequence[int], heads: int, q_len: int, q_dtype: str,
                         kv_dtype: str, causal: bool, pool_slots: int, period: int = 40,
                         step: float = 3.0, q_level: float = 4.0, name: str = "logit_jump") -> Case:
    """Inputs whose attention logits climb in large jumps along each row.

    Every query (token, head) has q[0:64] = q_level plus N(0, 0.05) noise and
    q[64:] = N(0, 0.05). Keys are N(0, 1), except that key j of a row with
    j % period == period // 2 (a "hot" key) has k[0:64] = step * (j // period + 1),
    and the key after it the same minus 0.05 (so the softmax mixes two keys).
    The n-th hot key of a row thus scores about 64 * q_level * step * n above
    an ordinary one: with the defaults and the softmax scale 1/sqrt(192),
    about 80 * n in base 2, so any later tile holding a hot key beats the
    first tile of its split by far more than its first-tile maximum.

    Draw order: a slot permutation (rows take consecutive runs of it), pool
    values, Q values; then the hot keys are written over their slots and
    everything is stored (bf16 by RNE, fp8 with a per-tensor scale)."""
    rng = np.random.default_rng(seed)
    lens = np.asarray(kv_lens, dtype=np.int64)
    rows = int(lens.shape[0])
    total = int(lens.sum())
    if total > pool_slots:
        raise ValueError("pool too small")
    perm = rng.permutation(pool_slots).astype(np.int64)
    pool = rng.standard_normal((pool_slots, D_LATENT), dtype=np.float32)
    T = rows * q_len
    q = (0.05 * rng.standard_normal((T, heads, D_LATENT))).astype(np.float32)
    q[:, :, :64] += np.float32(q_level)
    kv_indptr = np.zeros(rows + 1, dtype=np.int32)
    kv_indptr[1:] = np.cumsum(lens)
    kv_indices = perm[:total].astype(np.int32)
    for b in range(rows):
        base = int(kv_indptr[b])
        for j in range(int(lens[b])):
            if j % period == period // 2:
                level = np.float32(step * (j // period + 1))
                pool[kv_indices[base + j], :64] = level
                if j + 1 < int(lens[b]):
                    pool[kv_indices[base + j + 1], :64] = level - np.float32(0.05)
    pool_codes, kv_scale = _store(pool, kv_dtype)
    q_codes, q_scale = _store(q, q_dtype)
    qo_indptr = (np.arange(rows + 1) * q_len).astype(np.int32)
    return Case(name=name, rows=rows, q_len=q_len, heads=heads, causal=causal, q_dtype=q_dtype,
                kv_dtype=kv_dtype, q_codes=q_codes, q_scale=q_scale, pool_codes=pool_codes,
                kv_scale=kv_scale, qo_indptr=qo_indptr, kv_indptr=kv_indptr, kv_indices=kv_indices,
                sm_scale=SM_SCALE)
