"""GPU parity of decode-context-parallel shards on one GPU (virtual shards):
rank r of W takes every W-th key of each row (global positions r, r+W, ...),
mla_decode_fwd_dcp masks on global positions, and mla_merge_shards combines
the W results. Each shard is compared with the oracle's shard, the merge with
the oracle's unsharded row; W = 1 must equal mla_decode_fwd bit for bit."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from oracle.attention import attend_row, gather_rows       # noqa: E402
from oracle.codecs import decode                            # noqa: E402
from oracle.dcp import shard_attend                         # noqa: E402
from tests.gpu_harness import LSE_TOL, O_TOL                # noqa: E402
from workloads import make_case                             # noqa: E402


@pytest.fixture(scope="module")
def mla():
    from tests.lib_build import ensure_built
    ensure_built()
    import paged_mla_decode_02_amd as m
    m.load_library()
    return m


def _shard_lists(case, world, rank):
    idx, lens = [], []
    for b in range(case.rows):
        lo, hi = int(case.kv_indptr[b]), int(case.kv_indptr[b + 1])
        part = np.asarray(case.kv_indices[lo:hi])[rank::world]
        idx.append(part)
        lens.append(len(part))
    indptr = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    flat = np.concatenate(idx).astype(np.int32) if sum(lens) else np.zeros(1, np.int32)
    return flat, indptr, np.array(lens, np.int32)


def _run_shard(mla, case, world, rank, dev, o, lse):
    flat, indptr, lens = _shard_lists(case, world, rank)
    words = mla.plan(lens, case.heads, case.q_len, case.kv_dtype)
    plan_dev = torch.from_numpy(words).cuda()
    ws = mla.alloc_workspace(words)
    glob = torch.from_numpy(np.asarray(case.kv_lens, np.int32)).cuda()
    mla.decode_fwd_dcp(dev["q"], case.q_dtype, dev["q_scale"], dev["kv_pool"], case.kv_dtype,
                       dev["kv_scale"], dev["qo_indptr"], torch.from_numpy(indptr).cuda(),
                       torch.from_numpy(flat).cuda(), words, plan_dev, case.rows, case.heads,
                       case.q_len, case.causal, float(case.sm_scale), o, lse, world, rank, glob, ws)


def _check(got_o, got_l, ref_o, ref_l, tol):
    assert not np.isnan(got_o).any() and not np.isnan(got_l).any()
    ninf = np.isneginf(ref_l)
    assert np.array_equal(np.isneginf(got_l), ninf)
    refmax = max(np.abs(ref_o).max(), 1e-30)
    assert np.abs(got_o - ref_o).max() <= tol * refmax
    if (~ninf).any():
        assert np.abs(got_l[~ninf] - ref_l[~ninf]).max() <= LSE_TOL


CASES = [("bf16", "bf16", True, 16), ("bf16", "fp8", True, 64), ("fp8", "fp8", False, 64),
         ("bf16", "bf16", False, 128)]


@pytest.mark.parametrize("world", [2, 4, 8])
@pytest.mark.parametrize("q_dtype,kv_dtype,causal,heads", CASES)
def test_dcp_shards_and_merge(mla, world, q_dtype, kv_dtype, causal, heads):
    lens = [37, 300, 1003, 5, 0, 2048, 8]
    case = make_case(60 + world, lens, heads=heads, q_len=8, q_dtype=q_dtype, kv_dtype=kv_dtype,
                     causal=causal, pool_slots=8192, name=f"dcp{world}")
    print(f"dcp world={world} q={q_dtype} kv={kv_dtype} causal={causal} heads={heads}", flush=True)
    dev = mla.device_inputs(case.q_codes, case.q_scale, case.pool_codes, case.kv_scale,
                            case.qo_indptr, case.kv_indptr, case.kv_indices)
    T, H = case.num_tokens, heads
    o_parts = torch.full((world, T, H, 512), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse_parts = torch.full((world, T, H), float("nan"), dtype=torch.float32, device="cuda")
    for r in range(world):
        _run_shard(mla, case, world, r, dev, o_parts[r], lse_parts[r])
    o = torch.full((T, H, 512), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((T, H), float("nan"), dtype=torch.float32, device="cuda")
    mla.merge_shards(o_parts, lse_parts, o, lse)
    torch.cuda.synchronize()
    tol = O_TOL["fp8"] if "fp8" in (q_dtype, kv_dtype) else O_TOL["bf16"]
    op, lp = o_parts.float().cpu().numpy(), lse_parts.cpu().numpy()
    om, lm = o.float().cpu().numpy(), lse.cpu().numpy()
    for b in range(case.rows):
        t0, t1 = int(case.qo_indptr[b]), int(case.qo_indptr[b + 1])
        q = decode(case.q_codes[t0:t1], q_dtype, case.q_scale)
        k = gather_rows(case.pool_codes, kv_dtype, case.kv_scale, case.kv_indptr, case.kv_indices, b)
        for r in range(world):
            ref_o, ref_l = shard_attend(q, k, world, r, causal, case.sm_scale)
            _check(op[r, t0:t1], lp[r, t0:t1], ref_o, ref_l, tol)
        ref_o, ref_l = attend_row(q, k, causal, case.sm_scale)
        _check(om[t0:t1], lm[t0:t1], ref_o, ref_l, tol)


def test_dcp_world_one_is_plain_decode(mla):
    case = make_case(70, [100, 2000, 33], heads=32, q_len=4, q_dtype="bf16", kv_dtype="bf16",
                     causal=True, pool_slots=4096, name="dcp1")
    dev = mla.device_inputs(case.q_codes, case.q_scale, case.pool_codes, case.kv_scale,
                            case.qo_indptr, case.kv_indptr, case.kv_indices)
    T = case.num_tokens
    o1 = torch.empty((T, 32, 512), dtype=torch.bfloat16, device="cuda")
    l1 = torch.empty((T, 32), dtype=torch.float32, device="cuda")
    _run_shard(mla, case, 1, 0, dev, o1, l1)
    o2 = torch.empty_like(o1)
    l2 = torch.empty_like(l1)
    dec = mla.MlaDecoder(32, 4, "bf16", "bf16", True, float(case.sm_scale))
    dec.run(dev, case.kv_lens, o2, l2)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1, l2)
