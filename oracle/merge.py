"""Split-KV partials and their log-sum-exp merge (oracle; test infrastructure).

Split-KV (ATOM pull request 2462, "Summary" part 1 and "Dependencies": a split
plan, then split and merge): each split k of a row attends over its own key
range and yields a partial (O_k, LSE_k) by the plain definition restricted to
those keys. The merge is

    LSE = lse_max + ln sum_k exp(LSE_k - lse_max),
    O   = sum_k exp(LSE_k - LSE) * O_k,

skipping splits whose LSE_k is -inf (no visible key); if every split is empty
the result is O = 0, LSE = -inf. In exact arithmetic this equals attending
over the whole row at once, which the tests check.
"""
import numpy as np

from .attention import D_V, visible_count
from .codecs import decode


def merge_partials(O_parts, LSE_parts):
    """O_parts [n, ..., 512], LSE_parts [n, ...] float64 -> (O, LSE)."""
    O_parts = np.asarray(O_parts, dtype=np.float64)
    LSE_parts = np.asarray(LSE_parts, dtype=np.float64)
    lse_max = LSE_parts.max(axis=0)
    finite = np.isfinite(lse_max)
    safe_max = np.where(finite, lse_max, 0.0)
    w = np.where(np.isfinite(LSE_parts), np.exp(LSE_parts - safe_max), 0.0)
    tot = w.sum(axis=0)
    LSE = np.where(finite, safe_max + np.log(np.where(finite, tot, 1.0)), -np.inf)
    weights = np.where(np.isfinite(LSE_parts), np.exp(LSE_parts - np.where(finite, LSE, 0.0)), 0.0)
    O = (weights[..., None] * O_parts).sum(axis=0)
    O = np.where(finite[..., None], O, 0.0)
    return O, LSE


def attend_range(q_vals, k_vals, L, causal, sm_scale, begin, end):
    """Partial over keys [begin, end) of a row of L keys, same visibility rule
    as the whole row (token i sees keys j <= L - q_b + i when causal)."""
    q_b, H, D = q_vals.shape
    sigma = np.float64(np.float32(sm_scale))
    O = np.zeros((q_b, H, D_V))
    LSE = np.full((q_b, H), -np.inf)
    if end <= begin or q_b == 0:
        return O, LSE
    kr = k_vals[begin:end]
    scores = sigma * (q_vals.reshape(q_b * H, D) @ kr.T).reshape(q_b, H, end - begin)
    for i in range(q_b):
        last = visible_count(L, q_b, i, causal)   # keys 0..last-1 visible
        n = min(max(last - begin, 0), end - begin)
        if n == 0:
            continue
        s = scores[i, :, :n]
        m = s.max(axis=1, keepdims=True)
        lse = m[:, 0] + np.log(np.exp(s - m).sum(axis=1))
        LSE[i] = lse
        O[i] = np.exp(s - lse[:, None]) @ kr[:n, :D_V]
    return O, LSE


def split_attend(case, ranges_per_row, rows=None):
    """Attend each row split by ``ranges_per_row[b]`` (list of (begin, end)),
    merge, and return {b: (O_b, LSE_b, parts)}."""
    out = {}
    R = case.rows
    for b in (range(R) if rows is None else rows):
        t0, t1 = int(case.qo_indptr[b]), int(case.qo_indptr[b + 1])
        q = decode(case.q_codes[t0:t1], case.q_dtype, case.q_scale)
        lo, hi = int(case.kv_indptr[b]), int(case.kv_indptr[b + 1])
        k = decode(case.pool_codes[np.asarray(case.kv_indices[lo:hi], np.int64)],
                   case.kv_dtype, case.kv_scale)
        parts = [attend_range(q, k, hi - lo, case.causal, case.sm_scale, a, e)
                 for (a, e) in ranges_per_row[b]]
        O, LSE = merge_partials([p[0] for p in parts], [p[1] for p in parts])
        out[b] = (O, LSE, parts)
    return out
