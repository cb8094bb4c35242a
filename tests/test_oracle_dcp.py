"""Pins for the oracle's DCP shard attention (CPU only): W round-robin shards
merged by LSE equal attending over the whole row; one shard is the plain
definition; a brute force with explicit positions agrees."""
import math

import numpy as np
import pytest

from oracle.attention import attend_row
from oracle.dcp import attend_positions, shard_attend, shard_keys
from oracle.merge import merge_partials


def _row(rng, P, q_b, H):
    return rng.normal(0, 1, (q_b, H, 576)), rng.normal(0, 1, (P, 576))


@pytest.mark.parametrize("world", [1, 2, 3, 8])
@pytest.mark.parametrize("causal", [True, False])
def test_shards_merged_equal_unsharded(world, causal):
    rng = np.random.default_rng(world * 10 + causal)
    for P, q_b in [(37, 4), (5, 8), (64, 1), (9, 9)]:
        q, k = _row(rng, P, q_b, 3)
        parts = [shard_attend(q, k, world, r, causal, 0.07) for r in range(world)]
        O, LSE = merge_partials([p[0] for p in parts], [p[1] for p in parts])
        O_ref, LSE_ref = attend_row(q, k, causal, 0.07)
        fin = np.isfinite(LSE_ref)
        assert (np.isfinite(LSE) == fin).all()
        assert np.allclose(LSE[fin], LSE_ref[fin], atol=1e-12, rtol=0)
        assert np.allclose(O, O_ref, atol=1e-12, rtol=0)


def test_one_shard_is_the_plain_definition():
    rng = np.random.default_rng(3)
    q, k = _row(rng, 50, 8, 4)
    for causal in (True, False):
        O, LSE = shard_attend(q, k, 1, 0, causal, 0.1)
        O_ref, LSE_ref = attend_row(q, k, causal, 0.1)
        assert np.allclose(LSE, LSE_ref, atol=1e-12, rtol=0) and np.allclose(O, O_ref, atol=1e-12, rtol=0)


def test_shard_key_positions():
    assert list(shard_keys(10, 4, 1)) == [1, 5, 9]
    assert list(shard_keys(10, 4, 3)) == [3, 7]
    assert list(shard_keys(2, 4, 3)) == []


def test_positions_brute_force():
    rng = np.random.default_rng(4)
    q = rng.normal(0, 1, (3, 2, 576))
    k = rng.normal(0, 1, (5, 576))
    key_pos = np.array([2, 6, 10, 14, 18])
    query_pos = np.array([5, 14, 1])
    O, LSE = attend_positions(q, k, key_pos, query_pos, True, 0.05)
    for i in range(3):
        for h in range(2):
            vis = [j for j in range(5) if key_pos[j] <= query_pos[i]]
            if not vis:
                assert LSE[i, h] == -math.inf and not O[i, h].any()
                continue
            sigma = float(np.float32(0.05))   # the caller's float32 scale, widened
            s = [sigma * math.fsum(q[i, h] * k[j]) for j in vis]
            m = max(s)
            tot = math.fsum(math.exp(x - m) for x in s)
            assert abs(LSE[i, h] - (m + math.log(tot))) < 1e-12
            want = sum(math.exp(s[a] - m) / tot * k[j, :512] for a, j in enumerate(vis))
            assert np.allclose(O[i, h], want, atol=1e-12)
