"""In-kernel split merge and graph replay (GPU): split counters return to zero
after every call, repeated calls are bit-identical, and a decode captured in
a HIP graph with a UNIFORM plan built once replays correctly after the index
lists are rewritten in place with new (shorter) lengths."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from oracle.attention import attend_case                  # noqa: E402
from tests.gpu_harness import assert_parity                # noqa: E402
from workloads import make_case                            # noqa: E402


@pytest.fixture(scope="module")
def mla():
    from tests.lib_build import ensure_built
    ensure_built()
    import paged_mla_decode_02_amd as m
    m.load_library()
    return m


def _outputs(T, H):
    o = torch.full((T, H, 512), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((T, H), float("nan"), dtype=torch.float32, device="cuda")
    return o, lse


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
def test_repeated_calls_keep_counters_zero(mla, kv_dtype):
    """In-kernel merge (MLA_PLAN_MERGE_IN_KERNEL): the counters return to zero."""
    case = make_case(80, [3000, 100, 2500, 7, 0], heads=32, q_len=4, q_dtype="bf16", kv_dtype=kv_dtype,
                     causal=True, pool_slots=8192, name="repeat")
    print(f"repeat kv={kv_dtype}", flush=True)
    words = mla.plan(case.kv_lens, 32, 4, kv_dtype, mla.PLAN_UNIFORM | mla.PLAN_MERGE_IN_KERNEL)
    assert int(words[14]) > case.rows          # header word 14: S, the rows really are split
    dev = mla.device_inputs(case.q_codes, case.q_scale, case.pool_codes, case.kv_scale,
                            case.qo_indptr, case.kv_indptr, case.kv_indices)
    plan_dev = torch.from_numpy(words).cuda()
    ws = mla.alloc_workspace(words)
    results = []
    for _ in range(3):
        o, lse = _outputs(case.num_tokens, 32)
        mla.decode_fwd(dev["q"], "bf16", None, dev["kv_pool"], kv_dtype, dev["kv_scale"], dev["qo_indptr"],
                       dev["kv_indptr"], dev["kv_indices"], words, plan_dev, case.rows, 32, 4, True,
                       float(case.sm_scale), o, lse, ws)
        torch.cuda.synchronize()
        results.append((o.clone(), lse.clone()))
        assert int(ws[:256 * 1024].view(torch.int32).abs().sum().item()) == 0   # counters back to zero
    for o, lse in results[1:]:
        assert torch.equal(o.view(torch.int16), results[0][0].view(torch.int16))
        assert torch.equal(lse, results[0][1])
    assert_parity(case, results[0][0].float().cpu().numpy(), results[0][1].cpu().numpy())


@pytest.mark.parametrize("in_kernel", [False, True])
@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
def test_graph_replay_with_changing_lengths(mla, kv_dtype, in_kernel):
    H, QL, R = 16, 4, 4
    max_lens = np.array([3000, 2000, 1000, 500], np.int32)
    pool_slots = 16384
    base = make_case(81, max_lens, heads=H, q_len=QL, q_dtype="bf16", kv_dtype=kv_dtype, causal=True,
                     pool_slots=pool_slots, name="graph")
    print(f"graph kv={kv_dtype} in_kernel={in_kernel}", flush=True)
    flag = mla.PLAN_MERGE_IN_KERNEL if in_kernel else 0
    words = mla.plan(max_lens, H, QL, kv_dtype, mla.PLAN_UNIFORM | flag)   # built once, for the longest rows
    dev = mla.device_inputs(base.q_codes, base.q_scale, base.pool_codes, base.kv_scale,
                            base.qo_indptr, base.kv_indptr, base.kv_indices)
    plan_dev = torch.from_numpy(words).cuda()
    ws = mla.alloc_workspace(words)
    kv_indptr = dev["kv_indptr"].clone()
    kv_indices = torch.zeros(int(max_lens.sum()), dtype=torch.int32, device="cuda")
    o, lse = _outputs(base.num_tokens, H)

    def call():
        mla.decode_fwd(dev["q"], "bf16", None, dev["kv_pool"], kv_dtype, dev["kv_scale"], dev["qo_indptr"],
                       kv_indptr, kv_indices, words, plan_dev, R, H, QL, True, float(base.sm_scale), o, lse, ws)

    rng = np.random.default_rng(82)

    def load_lengths(lens):
        lens = np.asarray(lens, np.int32)
        indptr = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
        idx = rng.permutation(pool_slots)[:int(lens.sum())].astype(np.int32)
        kv_indptr.copy_(torch.from_numpy(indptr))
        kv_indices[:idx.shape[0]].copy_(torch.from_numpy(idx))
        return indptr, idx

    load_lengths(max_lens)
    call()                                  # eager warm-up
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()
    for lens in ([3000, 2000, 1000, 500], [1, 1999, 0, 257], [2999, 5, 700, 500], [64, 64, 64, 64]):
        indptr, idx = load_lengths(lens)
        o.fill_(float("nan"))
        lse.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        case = make_case(81, max_lens, heads=H, q_len=QL, q_dtype="bf16", kv_dtype=kv_dtype, causal=True,
                         pool_slots=pool_slots, name="graph")
        case.kv_indptr, case.kv_indices = indptr, idx
        assert_parity(case, o.float().cpu().numpy(), lse.cpu().numpy())
        if in_kernel:
            assert int(ws[:256 * 1024].view(torch.int32).abs().sum().item()) == 0
        # unrelated eager work between replays
        x = torch.randn(1 << 20, device="cuda")
        (x * 2).sum().item()


@pytest.mark.parametrize("name", ["draft_noncausal", "ragged_persistent_causal"])
def test_in_kernel_merge_workloads(mla, name):
    """The draft block (8 splits per row) and the ragged batch with the merge
    inside the decode kernel: same oracle bar as the default path."""
    from tests.gpu_harness import run_gpu
    from workloads import make_config
    case = make_config(name)
    dec = mla.MlaDecoder(case.heads, case.q_len, case.q_dtype, case.kv_dtype, case.causal,
                         float(case.sm_scale), mla.PLAN_AUTO | mla.PLAN_MERGE_IN_KERNEL)
    O, LSE, words = run_gpu(case, decoder=dec)
    rows = [0, case.rows // 2, case.rows - 1]
    assert_parity(case, O, LSE, rows)
