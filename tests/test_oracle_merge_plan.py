"""Pins for the oracle's split merge and split plan (CPU only)."""
import json
import os

import numpy as np
import pytest

from oracle.attention import attend_case
from oracle.merge import merge_partials, split_attend
from oracle.plan import (plan_ref, unpack_plan, MODE_AUTO, MODE_UNIFORM, MODE_LENGTH_AWARE,
                         KV_BF16, KV_FP8, N_MAX, OCC, XCDS, M_UNIT, ITEM_OVERHEAD, MIN_SPLIT_KEYS)
from workloads import make_case, config_lengths, CONFIGS, BF16, FP8

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def random_ranges(rng, L, n):
    cuts = np.sort(rng.integers(0, L + 1, n - 1)) if n > 1 else np.array([], int)
    edges = [0] + [int(c) for c in cuts] + [L]
    return list(zip(edges[:-1], edges[1:]))


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("seed", range(4))
def test_split_then_merge_equals_unsplit(causal, seed):
    rng = np.random.default_rng(200 + seed)
    lens = [int(x) for x in rng.integers(0, 120, 4)]
    case = make_case(300 + seed, lens, heads=3, q_len=int(rng.integers(1, 6)), q_dtype=BF16,
                     kv_dtype=FP8, causal=causal, pool_slots=1024)
    ranges = [random_ranges(rng, L, int(rng.integers(1, 7))) for L in lens]
    ref = attend_case(case)
    got = split_attend(case, ranges)
    for b in range(case.rows):
        O, LSE, _ = got[b]
        assert np.array_equal(np.isneginf(LSE), np.isneginf(ref[b][1]))
        fin = np.isfinite(LSE)
        np.testing.assert_allclose(LSE[fin], ref[b][1][fin], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(O, ref[b][0], rtol=1e-11, atol=1e-12)


def test_merge_edge_cases():
    O = np.random.default_rng(0).standard_normal((3, 2, 512))
    LSE = np.array([[-np.inf, 1.0], [-np.inf, -np.inf], [-np.inf, 2.0]])
    Om, Lm = merge_partials(O, LSE)
    assert np.isneginf(Lm[0]) and (Om[0] == 0).all()
    w1, w3 = np.exp(1.0), np.exp(2.0)
    assert Lm[1] == pytest.approx(np.log(w1 + w3), rel=1e-14)
    np.testing.assert_allclose(Om[1], (w1 * O[0, 1] + w3 * O[2, 1]) / (w1 + w3), rtol=1e-13)
    # one split is the identity
    O1, L1 = merge_partials(O[:1, 1:], LSE[:1, 1:])
    assert np.array_equal(O1, O[0, 1:]) and np.array_equal(L1, LSE[0, 1:])


def _check_fixture(fname):
    g = json.load(open(os.path.join(GOLDEN, fname)))
    a = g["args"]
    words = plan_ref(a["kv_lens"], a["H"], a["q_len_max"], a["kv_dtype"], a["mode"], a["C"])
    d = unpack_plan(words)
    for key, val in g["expect"].items():
        assert d[key] == val, (key, d[key], val)
    auto = plan_ref(a["kv_lens"], a["H"], a["q_len_max"], a["kv_dtype"], MODE_AUTO, a["C"])
    assert unpack_plan(auto)["mode"] == g["auto_mode"]


def test_plan_fixture_uniform():
    _check_fixture("plan_uniform_c4_h16.json")


def test_plan_fixture_length_aware():
    _check_fixture("plan_length_aware_c4_h128.json")


def check_invariants(lens, H, q_len, kv_dtype, mode, C):
    d = unpack_plan(plan_ref(lens, H, q_len, kv_dtype, mode, C))
    R, S, W, G, u = d["R"], d["S"], d["W"], d["G"], d["u"]
    assert u == -(-(H * q_len) // M_UNIT)
    sp = d["split_indptr"]
    assert sp[0] == 0 and sp[-1] == S and all(sp[i] < sp[i + 1] for i in range(R))
    nsplit = [sp[i + 1] - sp[i] for i in range(R)]
    assert max(nsplit) <= N_MAX
    slot = 0
    for b in range(R):
        edges = []
        for s in range(sp[b], sp[b + 1]):
            assert d["split_row"][s] == b
            edges.append((d["split_begin"][s], d["split_end"][s]))
            if nsplit[b] > 1:
                assert d["split_part"][s] == slot
                slot += 1
            else:
                assert d["split_part"][s] == -1
        # ranges partition [0, L_b) in order
        assert edges[0][0] == 0 and edges[-1][1] == lens[b]
        assert all(edges[i][1] == edges[i + 1][0] for i in range(len(edges) - 1))
        assert all(e >= a for a, e in edges)
    assert d["P"] == slot
    assert W == S * u
    items = list(zip(d["item_split"], d["item_m"]))
    assert sorted(items) == [(s, m) for s in range(S) for m in range(u)]
    wi = d["work_indptr"]
    assert wi[0] == 0 and wi[-1] == W and all(wi[i] <= wi[i + 1] for i in range(G))
    if d["mode"] == MODE_UNIFORM:
        assert G == W and len(set(nsplit)) == 1
        assert S <= R * N_MAX
    else:
        assert G <= max(OCC * C, u)
        assert S <= R + OCC * C
        # lanes: u workgroups of one chiplet run the same splits (in id order),
        # member j taking M tile j; every split is in exactly one lane, and a
        # row is cut only into pieces of at least MIN_SPLIT_KEYS keys (except
        # its last piece)
        X = XCDS
        while X > 1 and (OCC * C) // X < u:
            X //= 2
        lanes = {}
        for g in range(G):
            its = items[wi[g]:wi[g + 1]]
            if not its:
                continue
            ms = {m for _, m in its}
            assert len(ms) == 1
            seq = tuple(s for s, _ in its)
            assert all(seq[i] < seq[i + 1] for i in range(len(seq) - 1))
            lanes.setdefault(seq, []).append((g, ms.pop()))
        for seq, members in lanes.items():
            assert sorted(m for _, m in members) == list(range(u))
            assert len({g % X for g, _ in members}) == 1
        assert sorted(s for seq in lanes for s in seq) == list(range(S))
        for b in range(R):
            for s in range(sp[b], sp[b + 1] - 1):
                assert d["split_end"][s] - d["split_begin"][s] >= MIN_SPLIT_KEYS
    return d


def test_plan_invariants_random():
    rng = np.random.default_rng(5)
    for t in range(300):
        R = int(rng.integers(1, 40))
        lens = [int(x) for x in rng.integers(0, 20000, R)]
        if t % 5 == 0:
            lens = [0] * R
        H = int(rng.integers(1, 129))
        q = int(rng.integers(1, 17))
        C = int(rng.integers(1, 300))
        mode = int(rng.integers(0, 3))
        check_invariants(lens, H, q, int(rng.integers(0, 2)), mode, C)


def test_plan_rejects_bad_arguments():
    for args in [([], 16, 1), ([5], 0, 1), ([5], 129, 1), ([5], 16, 0), ([5], 16, 17), ([-1], 16, 1)]:
        with pytest.raises(ValueError):
            plan_ref(args[0], args[1], args[2], KV_BF16, MODE_AUTO, 256)
    # the fp8 PV flag needs fp8 KV and a separate merge
    with pytest.raises(ValueError):
        plan_ref([5], 16, 1, KV_BF16, MODE_AUTO | 0x200, 256)
    with pytest.raises(ValueError):
        plan_ref([5], 16, 1, KV_FP8, MODE_UNIFORM | 0x300, 256)


def test_fp8_pv_flag_only_marks_the_mode_word():
    lens = config_lengths("ragged_persistent_causal")
    for mode in (MODE_AUTO, MODE_UNIFORM, MODE_LENGTH_AWARE):
        plain = plan_ref(lens, 128, 2, KV_FP8, mode, 256)
        flagged = plan_ref(lens, 128, 2, KV_FP8, mode | 0x200, 256)
        assert flagged[7] == plain[7] | 0x200
        assert np.array_equal(np.delete(flagged, 7), np.delete(plain, 7))


def _estimates_from_words(words, C):
    """The two duration estimates of the plan spec, recomputed from plan words
    (not from the planner's internals): a split costs its keys plus
    ITEM_OVERHEAD; a UNIFORM plan lasts max(its costliest split, cdiv(u times
    its total cost, OCC*C)), a LENGTH_AWARE plan as long as its busiest
    workgroup's items (an empty row's split taking no room)."""
    d = unpack_plan(words)
    cost = [e - b + ITEM_OVERHEAD for b, e in zip(d["split_begin"], d["split_end"])]
    if d["mode"] & 0xFF == MODE_UNIFORM:
        return max(max(cost), -(-d["u"] * sum(cost) // (OCC * C)))
    # an empty row's split takes no room in a lane
    wi = d["work_indptr"]
    return max(sum(cost[s] for s in d["item_split"][wi[g]:wi[g + 1]] if d["split_end"][s] > d["split_begin"][s])
               for g in range(d["G"]))


def test_auto_mode_takes_the_shorter_estimate():
    """AUTO equals the explicit mode whose plan is estimated shorter (ties to
    UNIFORM), on random lengths and on every workload."""
    rng = np.random.default_rng(77)
    cases = []
    for name, spec in CONFIGS.items():
        kv = KV_FP8 if spec["kv_dtype"] == FP8 else KV_BF16
        cases.append(([int(x) for x in config_lengths(name)], spec["heads"], spec["q_len"], kv, 256))
    for _ in range(300):
        R = int(rng.integers(1, 40))
        lens = [int(x) for x in np.clip(np.rint(np.exp(rng.normal(7.0, 1.5, R))) - 20, 0, 100000)]
        cases.append((lens, int(rng.integers(1, 129)), int(rng.integers(1, 17)), int(rng.integers(0, 2)),
                      int(rng.choice([4, 16, 64, 256, 304]))))
    for lens, H, q, kv, C in cases:
        e_u = _estimates_from_words(plan_ref(lens, H, q, kv, MODE_UNIFORM, C), C)
        e_la = _estimates_from_words(plan_ref(lens, H, q, kv, MODE_LENGTH_AWARE, C), C)
        want = MODE_LENGTH_AWARE if e_la < e_u else MODE_UNIFORM
        auto = plan_ref(lens, H, q, kv, MODE_AUTO, C)
        assert unpack_plan(auto)["mode"] == want, (lens[:6], H, q, C, e_u, e_la)
        assert np.array_equal(auto, plan_ref(lens, H, q, kv, want, C))


def test_auto_mode_on_the_workloads():
    """Under AUTO the tiny case runs one split per row and the equal-length
    draft and top-k batches a uniform split; the 128-head verify, the long
    rows and the ragged batch plan their lanes from the real lengths (the
    choices that also measure faster on the GPU)."""
    C = 256
    expect = {"tiny_causal": (MODE_UNIFORM, 1), "verify_causal": (MODE_LENGTH_AWARE, None),
              "draft_noncausal": (MODE_UNIFORM, 8), "longctx_split": (MODE_LENGTH_AWARE, None),
              "ragged_persistent_causal": (MODE_LENGTH_AWARE, None), "sparse_topk": (MODE_UNIFORM, 2)}
    for name, (mode, n) in expect.items():
        spec = CONFIGS[name]
        lens = [int(x) for x in config_lengths(name)]
        kv = KV_FP8 if spec["kv_dtype"] == FP8 else KV_BF16
        d = check_invariants(lens, spec["heads"], spec["q_len"], kv, MODE_AUTO, C)
        assert d["mode"] == mode, name
        if n is not None:
            assert d["S"] == n * len(lens), name


@pytest.mark.parametrize("name", ["verify_causal", "draft_noncausal", "longctx_split",
                                  "ragged_persistent_causal", "sparse_topk"])
def test_length_aware_lanes_are_balanced(name):
    """On the workload shapes with 256 CUs, every workgroup gets work and the
    busiest one's cost (keys + ITEM_OVERHEAD per split) is within 10% of the
    mean: the plan cuts the rows' concatenated keys into equal lanes."""
    spec = CONFIGS[name]
    lens = [int(x) for x in config_lengths(name)]
    d = check_invariants(lens, spec["heads"], spec["q_len"], KV_FP8, MODE_LENGTH_AWARE, 256)
    wi, its = d["work_indptr"], d["item_split"]
    costs = [sum(d["split_end"][s] - d["split_begin"][s] + ITEM_OVERHEAD for s in its[wi[g]:wi[g + 1]])
             for g in range(d["G"])]
    assert d["G"] == 256 and min(costs) > 0
    assert max(costs) <= 1.10 * (sum(costs) / len(costs))
