"""Pins for the oracle's attention definition (CPU only).

Each test ties the numpy oracle to something other than itself: a pure-Python
brute force, torch's scaled-dot-product attention with torch's own
lower-right causal mask, closed forms, a hand-worked example and invariants.
"""
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F
from torch.nn.attention.bias import causal_lower_right

from oracle.attention import attend_row, attend_case, visible_count
from oracle.brute import brute_force
from workloads import make_case, BF16, FP8

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rand_rows(rng, q_b, H, L):
    return rng.standard_normal((q_b, H, 576)), rng.standard_normal((L, 576))


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("causal", [False, True])
def test_brute_force_agrees(seed, causal):
    rng = np.random.default_rng(100 + seed)
    q_b = int(rng.integers(1, 5))
    H = int(rng.integers(1, 5))
    L = int(rng.integers(0, 41))
    q, k = rand_rows(rng, q_b, H, L)
    sigma = np.float32(0.07)
    O, LSE = attend_row(q, k, causal, sigma)
    Ob, LSEb = brute_force(q.tolist(), k.tolist(), causal, float(sigma))
    Ob, LSEb = np.array(Ob), np.array(LSEb)
    assert np.array_equal(np.isinf(LSE), np.isinf(LSEb))
    fin = np.isfinite(LSEb)
    np.testing.assert_allclose(LSE[fin], LSEb[fin], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(O, Ob, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("q_b,L", [(1, 50), (4, 50), (8, 8), (8, 200), (16, 33)])
@pytest.mark.parametrize("causal", [False, True])
def test_matches_torch_sdpa(q_b, L, causal):
    """torch's SDPA (float64) with torch's lower-right causal mask is a library
    routine that fixes both the softmax and the mask alignment."""
    rng = np.random.default_rng(q_b * 1000 + L)
    H = 6
    q, k = rand_rows(rng, q_b, H, L)
    sigma = np.float32(1 / math.sqrt(192))
    O, LSE = attend_row(q, k, causal, sigma)
    tq = torch.from_numpy(q).permute(1, 0, 2).unsqueeze(0)          # [1, H, q_b, 576]
    tk = torch.from_numpy(k).expand(1, H, L, 576)
    tv = torch.from_numpy(k[:, :512]).expand(1, H, L, 512)
    mask = causal_lower_right(q_b, L) if causal else None
    ref = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, scale=float(sigma))
    ref = ref[0].permute(1, 0, 2).numpy()
    np.testing.assert_allclose(O, ref, rtol=1e-10, atol=1e-12)
    # LSE against torch.logsumexp over torch's scores and torch's mask
    s = float(sigma) * torch.einsum("ihd,jd->hij", torch.from_numpy(q), torch.from_numpy(k))
    if causal:
        s = s.masked_fill(~causal_lower_right(q_b, L)._materialize(), -math.inf)
    lse_ref = torch.logsumexp(s, dim=-1).permute(1, 0).numpy()
    np.testing.assert_allclose(LSE, lse_ref, rtol=1e-12, atol=1e-12)


def test_golden_three_keys():
    g = json.load(open(os.path.join(GOLDEN, "attention_three_keys.json")))
    lookup = {"0": 0.0, "ln2": math.log(2.0), "ln3": math.log(3.0), "ln6": math.log(6.0)}
    k = np.zeros((3, 576))
    k[:, 0] = [lookup[x] for x in g["k_dim0"]]
    k[:, 1] = g["k_dim1"]
    k[:, 2] = g["k_dim2"]
    k[:, 575] = g["k_dim575"]
    q = np.zeros((1, 1, 576))
    q[0, 0, 0] = g["q_dim0"]
    O, LSE = attend_row(q, k, False, np.float32(g["sm_scale"]))
    e = g["expect"]
    assert O[0, 0, 1] == pytest.approx(e["O_dim1"], abs=1e-13)
    assert O[0, 0, 2] == pytest.approx(e["O_dim2"], abs=1e-13)
    assert np.abs(O[0, 0, 3:]).max() == 0.0
    assert LSE[0, 0] == pytest.approx(lookup[e["LSE"]], abs=1e-14)
    # causal, two tokens
    q2 = np.zeros((2, 1, 576))
    q2[:, 0, 0] = g["q_dim0"]
    O2, LSE2 = attend_row(q2, k, True, np.float32(g["sm_scale"]))
    c = e["causal_q2_token0"]
    assert O2[0, 0, 1] == pytest.approx(c["O_dim1"], abs=1e-13)
    assert LSE2[0, 0] == pytest.approx(lookup[c["LSE"]], abs=1e-14)
    assert O2[1, 0, 1] == pytest.approx(e["O_dim1"], abs=1e-13)


def test_visible_counts_by_hand():
    # 5 keys, block of 3: token i at position 5-3+i sees keys 0..2+i.
    assert [visible_count(5, 3, i, True) for i in range(3)] == [3, 4, 5]
    assert [visible_count(5, 3, i, False) for i in range(3)] == [5, 5, 5]
    # block longer than the KV: positions 2-4+i = -2, -1, 0, 1
    assert [visible_count(2, 4, i, True) for i in range(4)] == [0, 0, 1, 2]


def test_single_visible_key():
    rng = np.random.default_rng(7)
    q, k = rand_rows(rng, 3, 4, 5)
    O, LSE = attend_row(q, k[:1], False, np.float32(0.1))
    for i in range(3):
        for h in range(4):
            assert np.array_equal(O[i, h], k[0, :512])
            assert LSE[i, h] == pytest.approx(np.float64(np.float32(0.1)) * q[i, h] @ k[0], rel=1e-14)


def test_constant_scores_give_prefix_mean():
    """q's first 512 dims are zero and every key has the same 64 RoPE values,
    so all scores are equal: O_i = mean of V over exactly the visible prefix
    and LSE = s + ln(count)."""
    rng = np.random.default_rng(8)
    L, q_b, H = 20, 6, 3
    k = rng.standard_normal((L, 576))
    k[:, 512:] = rng.standard_normal(64)
    q = np.zeros((q_b, H, 576))
    q[:, :, 512:] = rng.standard_normal((q_b, H, 64))
    sigma = np.float64(np.float32(0.125))
    O, LSE = attend_row(q, k, True, np.float32(0.125))
    for i in range(q_b):
        cnt = L - q_b + i + 1          # positions 14..19 see 15..20 keys
        for h in range(H):
            s = sigma * q[i, h, 512:] @ k[0, 512:]
            np.testing.assert_allclose(O[i, h], k[:cnt, :512].mean(axis=0), rtol=1e-12, atol=1e-13)
            assert LSE[i, h] == pytest.approx(s + math.log(cnt), rel=1e-13, abs=1e-13)


def test_causal_q1_equals_noncausal():
    case = make_case(11, [1, 17, 300], heads=5, q_len=1, q_dtype=BF16, kv_dtype=BF16,
                     causal=True, pool_slots=1024)
    a = attend_case(case, causal=True)
    b = attend_case(case, causal=False)
    for r in a:
        assert np.array_equal(a[r][0], b[r][0]) and np.array_equal(a[r][1], b[r][1])


def test_mask_discrimination():
    """The method the non-causal page used: the right-mask reference is far
    from the wrong-mask one, so a kernel's mask choice is visible."""
    case = make_case(12, [64, 64], heads=4, q_len=8, q_dtype=BF16, kv_dtype=BF16,
                     causal=True, pool_slots=512)
    a = attend_case(case, causal=True)
    b = attend_case(case, causal=False)
    for r in a:
        d = np.abs(a[r][0] - b[r][0]).max() / np.abs(b[r][0]).max()
        assert d > 5e-2
        # the last token of a causal block sees everything
        assert np.allclose(a[r][0][-1], b[r][0][-1], rtol=0, atol=1e-13)


def test_noncausal_permutation_invariance():
    case = make_case(13, [40, 77], heads=3, q_len=4, q_dtype=FP8, kv_dtype=FP8,
                     causal=False, pool_slots=512)
    ref = attend_case(case)
    rng = np.random.default_rng(0)
    idx = case.kv_indices.copy()
    for b in range(case.rows):
        lo, hi = case.kv_indptr[b], case.kv_indptr[b + 1]
        idx[lo:hi] = rng.permutation(idx[lo:hi])
    case.kv_indices = idx
    got = attend_case(case)
    for r in ref:
        np.testing.assert_allclose(got[r][0], ref[r][0], rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(got[r][1], ref[r][1], rtol=1e-13, atol=1e-13)


def test_identical_rows_identical_outputs():
    case = make_case(14, [50, 50, 50], heads=2, q_len=2, q_dtype=BF16, kv_dtype=BF16,
                     causal=True, pool_slots=256, shared_slots=True)
    case.q_codes[2:4] = case.q_codes[0:2]
    case.q_codes[4:6] = case.q_codes[0:2]
    out = attend_case(case)
    assert np.array_equal(out[0][0], out[1][0]) and np.array_equal(out[0][0], out[2][0])


def test_empty_rows_and_negative_positions():
    case = make_case(15, [0, 3], heads=2, q_len=5, q_dtype=BF16, kv_dtype=BF16,
                     causal=True, pool_slots=64)
    out = attend_case(case)
    assert (out[0][0] == 0).all() and np.isneginf(out[0][1]).all()
    # row 1: L=3, q=5: tokens 0,1 have negative positions -> empty
    O, LSE = out[1]
    assert (O[:2] == 0).all() and np.isneginf(LSE[:2]).all()
    assert np.isfinite(LSE[2:]).all()


def test_offset_indptr_equals_plain():
    a = make_case(16, [30, 45], heads=3, q_len=2, q_dtype=BF16, kv_dtype=FP8,
                  causal=True, pool_slots=512)
    b = make_case(16, [30, 45], heads=3, q_len=2, q_dtype=BF16, kv_dtype=FP8,
                  causal=True, pool_slots=512, kv_indptr_offset=37)
    assert b.kv_indptr[0] == 37
    ra, rb = attend_case(a), attend_case(b)
    for r in ra:
        assert np.array_equal(ra[r][0], rb[r][0])


def test_fp8_scales_match_sdpa_on_decoded_values():
    case = make_case(17, [90], heads=4, q_len=3, q_dtype=FP8, kv_dtype=FP8,
                     causal=False, pool_slots=256)
    from oracle.codecs import e4m3fn_to_f64
    q = e4m3fn_to_f64(case.q_codes) * case.q_scale
    k = e4m3fn_to_f64(case.pool_codes[case.kv_indices.astype(np.int64)]) * case.kv_scale
    O = attend_case(case)[0][0]
    tq = torch.from_numpy(q).permute(1, 0, 2).unsqueeze(0)
    tk = torch.from_numpy(k).expand(1, 4, 90, 576)
    tv = torch.from_numpy(k[:, :512]).expand(1, 4, 90, 512)
    ref = F.scaled_dot_product_attention(tq, tk, tv, scale=float(np.float32(case.sm_scale)))
    np.testing.assert_allclose(O, ref[0].permute(1, 0, 2).numpy(), rtol=1e-10, atol=1e-12)
