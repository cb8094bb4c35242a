"""Decode-context-parallel (DCP) shards, by definition (oracle; test
infrastructure).

A verify pass (q > 1 tokens) over a round-robin DCP KV shard needs the causal
mask on global positions (ATOM pull request 2760, "Problem"): with W ranks,
rank r holds the keys whose global position is r, r + W, r + 2W, ..., so its
local key j sits at global position j * W + r. Query token i of a block of
q_b tokens in a row of P keys in total (over all ranks) sits at global
position P - q_b + i. Causal: local key j is visible iff
j * W + r <= P - q_b + i; non-causal: every local key. Each rank yields a
partial (O_r, LSE_r) by the plain definition over its visible keys; the W
partials are combined with the log-sum-exp merge (oracle.merge), which in exact
arithmetic equals attending over the whole row (the tests check this).
"""
import numpy as np

from .attention import D_V


def attend_positions(q_vals, k_vals, key_pos, query_pos, causal, sm_scale):
    """q_vals [q_b, H, 576], k_vals [n, 576] decoded and scaled; key_pos [n]
    and query_pos [q_b] global positions. Returns O [q_b, H, 512], LSE [q_b, H]."""
    q_b, H, D = q_vals.shape
    n = k_vals.shape[0]
    sigma = np.float64(np.float32(sm_scale))
    O = np.zeros((q_b, H, D_V))
    LSE = np.full((q_b, H), -np.inf)
    if n == 0 or q_b == 0:
        return O, LSE
    key_pos = np.asarray(key_pos, dtype=np.int64)
    scores = sigma * (q_vals.reshape(q_b * H, D) @ k_vals.T).reshape(q_b, H, n)
    for i in range(q_b):
        vis = key_pos <= query_pos[i] if causal else np.ones(n, bool)
        if not vis.any():
            continue
        s = scores[i][:, vis]
        m = s.max(axis=1, keepdims=True)
        lse = m[:, 0] + np.log(np.exp(s - m).sum(axis=1))
        LSE[i] = lse
        O[i] = np.exp(s - lse[:, None]) @ k_vals[vis, :D_V]
    return O, LSE


def shard_keys(L_global: int, world: int, rank: int) -> np.ndarray:
    """Global positions of the keys rank `rank` holds, in local order."""
    return np.arange(rank, L_global, world, dtype=np.int64)


def shard_attend(q_vals, k_vals_global, world, rank, causal, sm_scale):
    """Rank `rank`'s partial for one row: its round-robin share of the row's
    keys (k_vals_global [P, 576] in global order), the mask on global
    positions."""
    q_b = q_vals.shape[0]
    P = k_vals_global.shape[0]
    pos = shard_keys(P, world, rank)
    query_pos = P - q_b + np.arange(q_b)
    return attend_positions(q_vals, k_vals_global[pos], pos, query_pos, causal, sm_scale)
