"""GPU parity: the HIP path through the C ABI against the CPU oracle, on the
same seeded inputs. Run on an MI355X; skipped elsewhere."""
import numpy as np
import pytest

from oracle.attention import attend_case, gather_rows
from oracle.codecs import decode
from oracle.plan import unpack_plan
from tests.gpu_harness import run_gpu, assert_parity, compare, tolerance
from workloads import make_case, make_config, BF16, FP8

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def lib():
    import torch
    import paged_mla_decode_02_amd as mla
    assert torch.cuda.is_available()
    mla.load_library()     # raises if the HIP library was not built
    return mla


def bf16_bits_of(values: np.ndarray) -> np.ndarray:
    """Exact bf16 bit patterns of values that are bf16-representable."""
    f = values.astype(np.float32)
    assert np.array_equal(f.astype(np.float64), values)
    bits = f.view(np.uint32)
    assert not (bits & 0xFFFF).any()
    return (bits >> 16).astype(np.uint16)


# --------------------------------------------------------------------------
# Index gather, bit-exact

@pytest.mark.parametrize("kv_dtype", [BF16, FP8])
@pytest.mark.parametrize("offset", [0, 45])
def test_gather_bit_exact(lib, kv_dtype, offset):
    import torch
    lens = [0, 1, 31, 32, 33, 100, 257, 1000]
    case = make_case(21, lens, heads=16, q_len=1, q_dtype=BF16, kv_dtype=kv_dtype, causal=True,
                     pool_slots=8192, kv_indptr_offset=offset)
    if kv_dtype == FP8:
        # every finite e4m3fn code appears in the pool
        codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
        case.pool_codes[:4] = np.resize(codes, (4, 576))
        case.kv_indices[offset:offset + 4] = [0, 1, 2, 3]
    words = lib.plan(case.kv_lens, 16, 1, kv_dtype, lib.PLAN_UNIFORM, 64)
    assert unpack_plan(words)["S"] > len(lens)          # rows really are split
    dev = lib.device_inputs(case.q_codes, None, case.pool_codes, case.kv_scale, case.qo_indptr,
                            case.kv_indptr, case.kv_indices)
    plan_dev = torch.from_numpy(words).cuda()
    nnz = int(case.kv_indptr[-1] - case.kv_indptr[0])
    dense = torch.zeros((nnz, 576), dtype=torch.int16, device="cuda")
    lib.debug_gather(dev["kv_pool"], kv_dtype, dev["kv_indptr"], dev["kv_indices"], words, plan_dev,
                     case.rows, dense)
    torch.cuda.synchronize()
    got = dense.cpu().numpy().view(np.uint16)
    for b in range(case.rows):
        ref = gather_rows(case.pool_codes, kv_dtype, None, case.kv_indptr, case.kv_indices, b)
        lo = int(case.kv_indptr[b] - case.kv_indptr[0])
        assert np.array_equal(got[lo:lo + len(ref)], bf16_bits_of(ref)), f"row {b}"


# --------------------------------------------------------------------------
# Every workload at full size, every row compared with the oracle, under
# every plan the library offers: AUTO (the default), UNIFORM, LENGTH_AWARE,
# and LENGTH_AWARE / UNIFORM with the split merge inside the decode kernel.
# The benchmark times AUTO, so its path is among these.

WORKLOADS = ["tiny_causal", "verify_causal", "verify_causal_fp8kv", "draft_noncausal", "longctx_split",
             "ragged_persistent_causal", "ragged_persistent_noncausal", "sparse_topk"]
PLAN_MODES = {"auto": 0, "uniform": 1, "length_aware": 2, "uniform_merge": 1 | 0x100,
              "length_aware_merge": 2 | 0x100}
# fp8 PV products (fp8-KV workloads only)
FP8_PV_MODES = {"auto_fp8pv": 0x200, "uniform_fp8pv": 1 | 0x200, "length_aware_fp8pv": 2 | 0x200}
FP8_KV_WORKLOADS = ["verify_causal_fp8kv", "draft_noncausal", "longctx_split", "ragged_persistent_causal",
                    "ragged_persistent_noncausal", "sparse_topk"]
WORKLOAD_PLANS = [(n, p) for n in WORKLOADS for p in PLAN_MODES] + \
                 [(n, p) for n in FP8_KV_WORKLOADS for p in FP8_PV_MODES]

_WORKLOAD_CACHE = {}


def workload_and_reference(name):
    """The full-size case and the oracle's O / LSE of every row, computed once
    per workload (the parametrization keeps one workload's tests together)."""
    if name not in _WORKLOAD_CACHE:
        _WORKLOAD_CACHE.clear()
        case = make_config(name)
        _WORKLOAD_CACHE[name] = (case, attend_case(case))
    return _WORKLOAD_CACHE[name]


@pytest.mark.parametrize("name,plan", WORKLOAD_PLANS)
def test_workload_parity(lib, name, plan):
    print(f"workload {name} plan {plan}", flush=True)
    case, ref = workload_and_reference(name)
    O, LSE, words = run_gpu(case, mode={**PLAN_MODES, **FP8_PV_MODES}[plan])
    info = unpack_plan(words)
    ratio, lse_err = assert_parity(case, O, LSE, ref=ref)
    assert len(ref) == case.rows                      # every row was compared
    print(f"{name} [{plan}]: err/max={ratio:.2e} lse_err={lse_err:.2e} S={info['S']} G={info['G']} "
          f"P={info['P']}")


# --------------------------------------------------------------------------
# Shapes, dtypes, masks and plans on small inputs (full oracle check)

SMALL = [
    # (heads, q_len, q_dtype, kv_dtype, causal, lens, mode, num_cus)
    (16, 1, BF16, BF16, True, [37, 128], 0, 256),
    (1, 1, BF16, BF16, True, [1, 2, 300], 0, 256),
    (8, 4, BF16, BF16, True, [0, 5, 64, 65, 700], 0, 256),
    (12, 3, BF16, FP8, False, [33, 31, 1000], 0, 256),
    (24, 16, BF16, BF16, True, [16, 17, 400], 0, 256),
    (32, 2, FP8, FP8, True, [90, 3, 2048], 0, 256),
    (64, 8, FP8, FP8, False, [512, 1023], 0, 256),
    (96, 5, FP8, BF16, True, [200, 7, 1500], 0, 256),
    (128, 1, BF16, FP8, True, [4000, 50, 0, 9000], 1, 256),         # uniform, many splits
    (128, 2, BF16, FP8, False, [4000, 50, 0, 9000] * 4, 2, 256),    # length-aware
    (128, 8, BF16, BF16, True, [2048, 100], 1, 256),
    (128, 16, BF16, BF16, True, [3, 20, 5000], 1, 16),               # q_len > L for row 0
    (7, 9, BF16, FP8, True, [1, 0, 9], 1, 2),                        # heads not a multiple of 16
    (16, 1, BF16, BF16, True, [40000], 1, 256),                      # uniform, 157 splits in one row
    (16, 1, BF16, FP8, False, [60000, 100], 2, 256),                 # lanes: about 250 splits in one row
]


# The fp8-KV cases again with fp8 PV products: items of one tile, odd and even
# tile counts (the last PV product covers one or two tiles), empty rows and
# splits, q_len above L, heads not a multiple of 16.
SMALL += [(H, q, qd, kd, c, lens, mode | 0x200, C) for (H, q, qd, kd, c, lens, mode, C) in SMALL if kd == FP8]
SMALL += [
    (16, 1, BF16, FP8, True, [1, 31, 32, 33, 63, 64, 65, 95, 96, 97], 1 | 0x200, 1),   # 1..4 tiles, unsplit
    (128, 4, FP8, FP8, False, [32 * k + 5 for k in range(12)], 2 | 0x200, 256),
]


@pytest.mark.parametrize("cfg", SMALL, ids=lambda c: f"h{c[0]}q{c[1]}{c[2]}{c[3]}{'c' if c[4] else 'n'}m{c[6]}")
def test_small_parity(lib, cfg):
    H, q, qd, kd, causal, lens, mode, C = cfg
    case = make_case(1000 + H * 17 + q, lens, heads=H, q_len=q, q_dtype=qd, kv_dtype=kd,
                     causal=causal, pool_slots=max(4096, 2 * sum(lens)))
    O, LSE, words = run_gpu(case, mode=mode, num_cus=C)
    assert_parity(case, O, LSE)


@pytest.mark.parametrize("heads", [1, 8, 12, 16, 24, 32, 64, 96, 128])
def test_head_sweep(lib, heads):
    case = make_case(50 + heads, [300, 77], heads=heads, q_len=2, q_dtype=BF16, kv_dtype=BF16,
                     causal=True, pool_slots=4096)
    O, LSE, _ = run_gpu(case)
    assert_parity(case, O, LSE)


@pytest.mark.parametrize("q_len", list(range(1, 17)))
@pytest.mark.parametrize("kv_dtype", [BF16, FP8])
def test_block_length_sweep(lib, q_len, kv_dtype):
    # includes the fp8 2-token block
    case = make_case(80 + q_len, [q_len + 5, 130], heads=16, q_len=q_len, q_dtype=BF16,
                     kv_dtype=kv_dtype, causal=(q_len % 2 == 0), pool_slots=4096)
    O, LSE, _ = run_gpu(case)
    assert_parity(case, O, LSE)


def test_query_row_magnitudes_fp8_kv(lib):
    """bf16 queries against fp8 KV: the decode splits each query row into two
    fp8 operands (a high and a low part) under a power-of-two scale taken from
    the row's largest element. Rows far from unit size, rows whose elements
    span 24 binades, all-zero rows, rows of bf16 subnormals and rows with one
    nonzero element must still match the oracle."""
    case = make_case(95, [300, 77, 40], heads=16, q_len=3, q_dtype=BF16, kv_dtype=FP8, causal=True,
                     pool_slots=4096)
    rng = np.random.default_rng(95)
    q = (case.q_codes.astype(np.uint32) << 16).view(np.float32).astype(np.float64).reshape(-1, 576)
    for i in range(q.shape[0]):
        kind = i % 8
        if kind == 0:
            q[i] *= 2.0 ** -30
        elif kind == 1:
            q[i] *= 2.0 ** -12
        elif kind == 2:
            q[i] *= 8.0
        elif kind == 3:
            q[i] *= 2.0 ** rng.integers(-24, 1, 576)
        elif kind == 4:
            q[i] = 0.0
        elif kind == 5:
            q[i] = rng.integers(-127, 128, 576) * 2.0 ** -133     # bf16 subnormals
        elif kind == 6:
            q[i] = 0.0
            q[i, rng.integers(0, 576)] = 1.5
    case.q_codes = bf16_bits_of(q).reshape(case.q_codes.shape)
    O, LSE, _ = run_gpu(case)
    ratio, lse_err = assert_parity(case, O, LSE)
    print(f"max|err|/max|O_ref| {ratio:.2e}, max|dLSE| {lse_err:.2e}")


def test_ragged_blocks_and_offset_indptr(lib):
    case = make_case(91, [40, 0, 300, 17, 5], heads=16, q_len=6, q_dtype=BF16, kv_dtype=FP8,
                     causal=True, pool_slots=4096, q_lens=[6, 2, 0, 6, 1], kv_indptr_offset=13)
    O, LSE, _ = run_gpu(case, mode=1, num_cus=8)
    assert_parity(case, O, LSE)


def test_forced_split_matches_unsplit(lib):
    case = make_case(92, [6000, 3000], heads=64, q_len=2, q_dtype=BF16, kv_dtype=BF16,
                     causal=True, pool_slots=16384)
    O1, L1, w1 = run_gpu(case, mode=1, num_cus=1)       # one split per row
    O2, L2, w2 = run_gpu(case, mode=1, num_cus=256)     # many splits + merge
    assert unpack_plan(w1)["S"] == 2 and unpack_plan(w2)["S"] > 2
    ref = attend_case(case)
    assert_parity(case, O1, L1, ref=ref)
    assert_parity(case, O2, L2, ref=ref)
    assert np.abs(O1 - O2).max() <= 1e-2 * np.abs(O1).max()


@pytest.mark.parametrize("n", [2, 3, 4, 5, 8, 9, 16, 17, 40])
def test_merge_split_counts(lib, n):
    """Every chunk size of the split merge (2, 4 and 8 splits per round trip,
    one or two chunks) and the wide merge beyond 16 splits: a UNIFORM plan
    cuts each row of 256 n keys into n splits of 256."""
    case = make_case(300 + n, [256 * n, 256 * n - 77], heads=16, q_len=2, q_dtype=BF16, kv_dtype=BF16,
                     causal=True, pool_slots=max(4096, 600 * n))
    O, LSE, words = run_gpu(case, mode=1, num_cus=256)
    info = unpack_plan(words)
    assert info["S"] == 2 * n          # n splits in each of the two rows
    assert_parity(case, O, LSE)


@pytest.mark.parametrize("qd,kd,mode", [(BF16, BF16, 1), (BF16, FP8, 1), (FP8, FP8, 1), (FP8, BF16, 1),
                                         (BF16, FP8, 0x201), (FP8, FP8, 0x201)],
                         ids=["bf16-bf16", "bf16-fp8", "fp8-fp8", "fp8-bf16", "bf16-fp8-pv8", "fp8-fp8-pv8"])
@pytest.mark.parametrize("causal", [True, False])
def test_one_and_two_tile_items(lib, qd, kd, mode, causal):
    """Items of one, two and three 32-key tiles (the prologue's one-tile and
    two-tile wait counts, and the last-step paths), for every dtype pair and
    both masks: rows of 1 .. 96 keys, one split each."""
    lens = [1, 5, 31, 32, 33, 63, 64, 65, 96]
    case = make_case(9100 + 7 * len(qd) + len(kd) + (mode >> 9) + 2 * causal, lens, heads=16, q_len=4,
                     q_dtype=qd, kv_dtype=kd, causal=causal, pool_slots=4096)
    O, LSE, words = run_gpu(case, mode=mode, num_cus=1)
    assert unpack_plan(words)["S"] == len(lens)
    assert_parity(case, O, LSE)


def _random_shape(k):
    """Seeded random shape k: heads, block length, dtypes, mask, row lengths
    (with empty rows), ragged query blocks, plan mode and CU count."""
    rng = np.random.default_rng(7000 + k)
    H = int(rng.choice([1, 3, 8, 16, 20, 33, 64, 96, 127, 128]))
    q = int(rng.integers(1, 17))
    qd, kd = [(BF16, BF16), (BF16, FP8), (FP8, FP8), (FP8, BF16)][k % 4]
    rows = int(rng.integers(1, 6))
    lens = [int(x) for x in rng.integers(0, 1500, rows)]
    if rng.random() < 0.3:
        lens[int(rng.integers(rows))] = 0
    q_lens = [int(x) for x in rng.integers(0, q + 1, rows)] if rng.random() < 0.5 else None
    mode = int(rng.choice([0, 1, 2]))
    if kd == FP8 and rng.random() < 0.4:
        mode |= 0x200
    C = int(rng.choice([1, 4, 32, 256]))
    return H, q, qd, kd, bool(rng.random() < 0.6), lens, q_lens, mode, C


@pytest.mark.parametrize("k", range(48))
def test_random_shapes(lib, k):
    """A seeded sweep of shapes no other test picks by hand, each compared with
    the oracle on every row."""
    H, q, qd, kd, causal, lens, q_lens, mode, C = _random_shape(k)
    case = make_case(8000 + k, lens, heads=H, q_len=q, q_dtype=qd, kv_dtype=kd, causal=causal,
                     pool_slots=max(4096, 2 * sum(lens)), q_lens=q_lens)
    O, LSE, words = run_gpu(case, mode=mode, num_cus=C)
    print(f"random shape {k}: H={H} q={q} {qd}/{kd} causal={causal} lens={lens} q_lens={q_lens} "
          f"mode={mode:#x} C={C} S={unpack_plan(words)['S']}")
    assert_parity(case, O, LSE)


def test_all_empty_inputs(lib):
    """Every row without keys (an empty index list), and every query block
    empty (no query tokens at all): the first gives O = 0 and LSE = -inf for
    every token, the second writes nothing."""
    case = make_case(95, [0, 0, 0], heads=16, q_len=4, q_dtype=BF16, kv_dtype=FP8, causal=True,
                     pool_slots=4096)
    O, LSE, _ = run_gpu(case, mode=1, num_cus=8)
    assert (O == 0).all() and np.isneginf(LSE).all()
    case = make_case(96, [100, 0, 300], heads=16, q_len=4, q_dtype=BF16, kv_dtype=BF16, causal=True,
                     pool_slots=4096, q_lens=[0, 0, 0])
    O, LSE, _ = run_gpu(case, mode=2, num_cus=8)
    assert O.shape[0] == 0 and LSE.shape[0] == 0


def test_mask_discrimination(lib):
    """The kernel runs the mask that was asked for: close to the right-mask
    reference, far from the wrong one (the check the non-causal draft page
    reports)."""
    for causal in (True, False):
        case = make_case(93, [64, 200], heads=16, q_len=8, q_dtype=BF16, kv_dtype=FP8,
                         causal=causal, pool_slots=4096)
        O, LSE, _ = run_gpu(case)
        right, _ = compare(case, O, LSE, ref=attend_case(case, causal=causal))
        wrong_ref = attend_case(case, causal=not causal)
        refmax = max(float(np.abs(v[0]).max()) for v in wrong_ref.values())
        wrong = max(float(np.abs(O[case.qo_indptr[b]:case.qo_indptr[b + 1]] - v[0]).max())
                    for b, v in wrong_ref.items()) / refmax
        assert right <= tolerance(case)
        assert wrong > 10 * right, (right, wrong)


def test_deterministic_and_identical_rows(lib):
    case = make_case(94, [500, 500, 500, 500], heads=16, q_len=4, q_dtype=BF16, kv_dtype=FP8,
                     causal=False, pool_slots=4096, shared_slots=True)
    for r in range(1, 4):
        case.q_codes[4 * r:4 * r + 4] = case.q_codes[0:4]
    O1, L1, _ = run_gpu(case)
    O2, L2, _ = run_gpu(case)
    assert np.array_equal(O1, O2) and np.array_equal(L1, L2)
    for r in range(1, 4):
        assert np.array_equal(O1[4 * r:4 * r + 4], O1[0:4])
        assert np.array_equal(L1[4 * r:4 * r + 4], L1[0:4])
    assert_parity(case, O1, L1)


def test_binding_refuses_bad_tensors(lib):
    """The Python binding checks every tensor before the C ABI sees a pointer:
    a uint8 pool declared bf16, a flattened pool, int64 index lists, short or
    mistyped outputs and a tensor on the CPU are refused; nothing runs."""
    import torch
    case = make_case(96, [40, 70], heads=16, q_len=2, q_dtype=BF16, kv_dtype=BF16, causal=True,
                     pool_slots=1024)
    dev = lib.device_inputs(case.q_codes, None, case.pool_codes, None, case.qo_indptr, case.kv_indptr,
                            case.kv_indices)
    words = lib.plan(case.kv_lens, 16, 2, BF16)
    plan_dev = torch.from_numpy(words).cuda()
    T = case.num_tokens
    good = dict(q=dev["q"], kv_pool=dev["kv_pool"], qo_indptr=dev["qo_indptr"], kv_indptr=dev["kv_indptr"],
                kv_indices=dev["kv_indices"],
                o=torch.full((T, 16, 512), float("nan"), dtype=torch.bfloat16, device="cuda"),
                lse=torch.full((T, 16), float("nan"), dtype=torch.float32, device="cuda"))

    def call(**over):
        a = dict(good, **over)
        lib.decode_fwd(a["q"], BF16, None, a["kv_pool"], BF16, None, a["qo_indptr"], a["kv_indptr"],
                       a["kv_indices"], words, plan_dev, case.rows, 16, 2, True, float(case.sm_scale),
                       a["o"], a["lse"])

    bad = [
        (TypeError, dict(kv_pool=dev["kv_pool"].view(torch.uint8))),          # bf16 pool as bytes
        (ValueError, dict(kv_pool=dev["kv_pool"].view(-1))),                  # flattened pool
        (TypeError, dict(kv_indptr=dev["kv_indptr"].long())),                 # int64 indptr
        (TypeError, dict(kv_indices=dev["kv_indices"].long())),
        (ValueError, dict(qo_indptr=dev["qo_indptr"][:-1])),                  # wrong length
        (ValueError, dict(o=good["o"][:T - 1])),                              # too few tokens
        (TypeError, dict(o=good["o"].float())),                               # not bf16
        (TypeError, dict(lse=good["lse"].double())),
        (ValueError, dict(q=dev["q"].view(T, 16 * 576))),                     # wrong shape
        (ValueError, dict(q=dev["q"].cpu())),                                 # not on the GPU
        (ValueError, dict(kv_pool=dev["kv_pool"][:, :288])),                  # not contiguous
    ]
    for exc, over in bad:
        with pytest.raises(exc):
            call(**over)
    torch.cuda.synchronize()
    assert torch.isnan(good["o"].float()).all()                               # nothing was written
    call()
    torch.cuda.synchronize()
    assert_parity(case, good["o"].float().cpu().numpy(), good["lse"].cpu().numpy())
