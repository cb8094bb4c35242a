"""mla_decode_fwd_noalloc (GPU): the decode with its split partials in the
library's static per-GPU scratch matches mla_decode_fwd with a caller
workspace bit for bit, on two calls in a row (the second smaller), and both
match the oracle. Covers a merge-kernel plan, an in-kernel-merge plan (its
counters are cleared by the call) and a plan with no split (no scratch)."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from oracle.plan import unpack_plan                        # noqa: E402
from tests.gpu_harness import assert_parity                # noqa: E402
from workloads import make_case                            # noqa: E402


@pytest.fixture(scope="module")
def mla():
    import paged_mla_decode_02_amd as m
    assert torch.cuda.is_available()
    m.load_library()
    return m


def _run(mla, case, words, noalloc):
    dev = mla.device_inputs(case.q_codes, case.q_scale, case.pool_codes, case.kv_scale,
                            case.qo_indptr, case.kv_indptr, case.kv_indices)
    plan_dev = torch.from_numpy(words).cuda()
    T, H = case.num_tokens, case.heads
    o = torch.full((T, H, 512), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((T, H), float("nan"), dtype=torch.float32, device="cuda")
    args = (dev["q"], case.q_dtype, dev["q_scale"], dev["kv_pool"], case.kv_dtype, dev["kv_scale"],
            dev["qo_indptr"], dev["kv_indptr"], dev["kv_indices"], words, plan_dev, case.rows, H,
            case.q_len, case.causal, float(case.sm_scale), o, lse)
    if noalloc:
        mla.decode_fwd_noalloc(*args)
    else:
        mla.decode_fwd(*args, workspace=mla.alloc_workspace(words))
    torch.cuda.synchronize()
    return o.view(torch.int16).cpu().numpy(), lse.cpu().numpy()


@pytest.mark.parametrize("mode", [1, 2, 1 | 0x100, 2 | 0x100], ids=["uniform", "length_aware",
                                                                     "uniform_merge", "length_aware_merge"])
@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
def test_noalloc_matches_workspace_call(mla, kv_dtype, mode):
    cases = [make_case(400, [9000, 300, 5000, 0, 4100], heads=64, q_len=4, q_dtype="bf16",
                       kv_dtype=kv_dtype, causal=True, pool_slots=32768, name="first"),
             make_case(401, [2500, 40, 700], heads=16, q_len=2, q_dtype="bf16",
                       kv_dtype=kv_dtype, causal=False, pool_slots=8192, name="second")]
    for case in cases:                        # two calls in a row, the second smaller
        print(f"noalloc {case.name} kv={kv_dtype} mode={mode:#x}", flush=True)
        words = mla.plan(case.kv_lens, case.heads, case.q_len, kv_dtype, mode)
        assert unpack_plan(words)["P"] > 0    # the call really uses the scratch
        assert 0 < mla.workspace_size(words) <= mla.NOALLOC_SCRATCH_BYTES
        o_ref, l_ref = _run(mla, case, words, noalloc=False)
        o, l = _run(mla, case, words, noalloc=True)
        assert np.array_equal(o, o_ref), "O differs from mla_decode_fwd"
        assert np.array_equal(l, l_ref, equal_nan=True), "LSE differs from mla_decode_fwd"
        of = (o.view(np.uint16).astype(np.uint32) << 16).view(np.float32)
        assert_parity(case, of.reshape(case.num_tokens, case.heads, 512), l)


def test_noalloc_unsplit_plan(mla):
    case = make_case(402, [37, 128], heads=16, q_len=1, q_dtype="bf16", kv_dtype="bf16", causal=True,
                     pool_slots=4096)
    words = mla.plan(case.kv_lens, 16, 1, "bf16", 1)
    assert mla.workspace_size(words) == 0
    o_ref, l_ref = _run(mla, case, words, noalloc=False)
    o, l = _run(mla, case, words, noalloc=True)
    assert np.array_equal(o, o_ref) and np.array_equal(l, l_ref)
