"""GPU parity where a row's logits climb by far more than the decode's
reference headroom after its first tile.

The decode kernel fixes each query row's reference maximum (base 2) at the
row's first visible key tile of 32 keys and accumulates O against it without
rescaling; a later tile whose maximum exceeds that reference by more than 64
makes the work item run again with every row's true maximum. The inputs here
(workloads.make_logit_jump_case) put "hot" keys of increasing size every 40
keys, so every split of more than a few tiles takes that second pass. The test
first proves, in float64 on the stored values, that the climb really exceeds
64 in base 2 inside each such split, then compares every row with the oracle.
It covers bf16 / bf16, bf16 Q with fp8 KV and fp8 / fp8; causal and
non-causal; unsplit rows, split rows merged by the merge kernel, split
rows merged inside the decode kernel, and (fp8 KV) the fp8 PV products."""
import math

import numpy as np
import pytest

from oracle.codecs import decode
from oracle.plan import unpack_plan
from tests.gpu_harness import run_gpu, assert_parity
from workloads import make_logit_jump_case, BF16, FP8

pytestmark = pytest.mark.gpu

TILE = 32          # keys per LDS tile of the decode kernel
HEADROOM = 64.0    # base-2 headroom above a row's reference maximum
LENS = [400, 300, 37, 130]
HEADS, Q_LEN = 16, 4

PLANS = {
    "unsplit": (1, 1),                   # UNIFORM on one CU: one split per row
    "split": (1, 256),                   # UNIFORM on 256 CUs: two splits per long row
    "split_merge_in_kernel": (1 | 0x100, 256),
    "unsplit_fp8pv": (1 | 0x200, 1),     # fp8 PV products (fp8 KV only)
    "split_fp8pv": (1 | 0x200, 256),
}


@pytest.fixture(scope="module", autouse=True)
def lib():
    import torch
    import paged_mla_decode_02_amd as mla
    assert torch.cuda.is_available()
    mla.load_library()
    return mla


def split_climbs(case, words):
    """For each split: the largest base-2 rise, over its (token, head) rows,
    of a later visible tile's maximum score above the first visible tile's.
    Float64 on the stored values."""
    plan = unpack_plan(words)
    sigma2 = float(np.float32(case.sm_scale)) * math.log2(math.e)
    out = []
    for s in range(plan["S"]):
        b, beg, end = plan["split_row"][s], plan["split_begin"][s], plan["split_end"][s]
        L = int(case.kv_indptr[b + 1] - case.kv_indptr[b])
        q_b = int(case.qo_indptr[b + 1] - case.qo_indptr[b])
        slots = case.kv_indices[case.kv_indptr[b] + beg:case.kv_indptr[b] + end]
        k = decode(case.pool_codes[slots], case.kv_dtype, case.kv_scale)
        q = decode(case.q_codes[case.qo_indptr[b]:case.qo_indptr[b + 1]], case.q_dtype, case.q_scale)
        scores = sigma2 * np.einsum("thd,jd->thj", q, k)     # [q_b, H, keys of the split]
        best = -np.inf
        for i in range(q_b):
            last = min(end - 1, L - q_b + i) if case.causal else end - 1
            n = last - beg + 1
            if n <= TILE:
                continue
            first = scores[i, :, :TILE].max(axis=1)
            later = scores[i, :, TILE:n].max(axis=1)
            best = max(best, float((later - first).max()))
        out.append((end - beg, best))
    return out


DTYPES = [(BF16, BF16), (BF16, FP8), (FP8, FP8)]
CASES = [pytest.param(d, c, p, id=f"q{d[0]}kv{d[1]}-{'causal' if c else 'noncausal'}-{p}")
         for d in DTYPES for c in (True, False) for p in PLANS
         if d[1] == FP8 or not PLANS[p][0] & 0x200]     # fp8 PV products need fp8 KV


@pytest.mark.parametrize("dtypes,causal,plan", CASES)
def test_logit_climb_rerun(lib, dtypes, causal, plan):
    q_dtype, kv_dtype = dtypes
    mode, cus = PLANS[plan]
    print(f"logit climb q={q_dtype} kv={kv_dtype} causal={causal} plan={plan}", flush=True)
    case = make_logit_jump_case(300, LENS, heads=HEADS, q_len=Q_LEN, q_dtype=q_dtype, kv_dtype=kv_dtype,
                                causal=causal, pool_slots=4096)
    words = lib.plan(case.kv_lens, HEADS, Q_LEN, kv_dtype, mode, cus)
    climbs = split_climbs(case, words)
    # every split of three tiles or more climbs past the headroom
    long_splits = [c for n, c in climbs if n >= 3 * TILE]
    assert long_splits and min(long_splits) > HEADROOM, climbs
    if not plan.startswith("unsplit"):
        assert unpack_plan(words)["S"] > case.rows          # the long rows really are split
    O, LSE, used = run_gpu(case, mode=mode, num_cus=cus)
    assert np.array_equal(used, words)
    ratio, lse_err = assert_parity(case, O, LSE)
    print(f"  climbs {[round(c, 1) for _, c in climbs]}  err/max={ratio:.2e} lse_err={lse_err:.2e}")
