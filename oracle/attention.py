"""Gathered-index MLA decode by its plain definition (oracle; test infrastructure).

For request row b with query tokens qo_indptr[b]..qo_indptr[b+1]-1 and keys
kv_indices[kv_indptr[b] .. kv_indptr[b+1]-1] (one flat page-size-1 list, one
row per request; vLLM pull request 53001, "Purpose"):

1. L = kv_indptr[b+1] - kv_indptr[b]; q_b = qo_indptr[b+1] - qo_indptr[b].
2. k_j = the stored latent row of slot kv_indices[kv_indptr[b] + j], decoded
   and times the per-tensor KV scale; 576 values, of which the first 512 are
   the compressed latent and the last 64 the RoPE part. V is k_j[:512]: MLA
   reads keys and values from the same latent row.
3. Query token i of the row, head h: q = decoded Q times the per-tensor Q scale.
4. Visible keys: the row's KV holds the committed context plus the q_b block
   tokens, so token i sits at global position L - q_b + i and key j at
   position j. Causal (the speculative verify pass; ATOM pull request 2760,
   "Problem": the mask applies on global positions): j <= L - q_b + i.
   Non-causal (the draft block; vLLM pull request 53001, "Purpose"): all j < L.
5. s_j = sigma * (q . k_j), sigma the caller's float32 softmax scale.
6. LSE = ln sum_{visible j} exp(s_j) (natural log, scale inside; the pages name
   an LSE output without defining its base), O = sum_j exp(s_j - LSE) v_j.
7. No visible key: O = 0 and LSE = -inf (rows with no KV, "K=0 padded rows"
   in ATOM pull request 2462, "Test plan"; empty splits; causal tokens whose
   position is negative).

Everything is float64; the row's scores are one matrix product (a library
primitive), the softmax is written out.
"""
import numpy as np

from .codecs import decode

D_LATENT = 576
D_V = 512


def visible_count(L: int, q_b: int, i: int, causal: bool) -> int:
    """Number of visible keys for token i (they are keys 0..count-1)."""
    if not causal:
        return L
    return int(min(max(L - q_b + i + 1, 0), L))


def attend_row(q_vals: np.ndarray, k_vals: np.ndarray, causal: bool, sm_scale):
    """q_vals [q_b, H, 576] and k_vals [L, 576], already decoded and scaled.

    Returns O [q_b, H, 512] and LSE [q_b, H], float64."""
    q_b, H, D = q_vals.shape
    L = k_vals.shape[0]
    sigma = np.float64(np.float32(sm_scale))
    O = np.zeros((q_b, H, D_V), dtype=np.float64)
    LSE = np.full((q_b, H), -np.inf, dtype=np.float64)
    if L == 0 or q_b == 0:
        return O, LSE
    scores = sigma * (q_vals.reshape(q_b * H, D) @ k_vals.T).reshape(q_b, H, L)
    for i in range(q_b):
        n = visible_count(L, q_b, i, causal)
        if n == 0:
            continue
        s = scores[i, :, :n]                       # [H, n]
        m = s.max(axis=1, keepdims=True)
        lse = m[:, 0] + np.log(np.exp(s - m).sum(axis=1))
        p = np.exp(s - lse[:, None])               # softmax weights
        LSE[i] = lse
        O[i] = p @ k_vals[:n, :D_V]
    return O, LSE


def gather_rows(pool_codes, kv_dtype, kv_scale, kv_indptr, kv_indices, b):
    lo, hi = int(kv_indptr[b]), int(kv_indptr[b + 1])
    slots = np.asarray(kv_indices[lo:hi], dtype=np.int64)
    return decode(pool_codes[slots], kv_dtype, kv_scale)


def attend(q_codes, q_dtype, q_scale, pool_codes, kv_dtype, kv_scale,
           qo_indptr, kv_indptr, kv_indices, causal, sm_scale, rows=None):
    """Decode every row in ``rows`` (default: all). Returns {b: (O_b, LSE_b)}
    with O_b [q_b, H, 512] and LSE_b [q_b, H]."""
    R = len(qo_indptr) - 1
    out = {}
    for b in (range(R) if rows is None else rows):
        t0, t1 = int(qo_indptr[b]), int(qo_indptr[b + 1])
        q = decode(q_codes[t0:t1], q_dtype, q_scale)
        k = gather_rows(pool_codes, kv_dtype, kv_scale, kv_indptr, kv_indices, b)
        out[b] = attend_row(q, k, causal, sm_scale)
    return out


def attend_case(case, rows=None, causal=None):
    """Convenience wrapper over a ``workloads.Case``-like object."""
    return attend(case.q_codes, case.q_dtype, case.q_scale, case.pool_codes,
                  case.kv_dtype, case.kv_scale, case.qo_indptr, case.kv_indptr,
                  case.kv_indices, case.causal if causal is None else causal,
                  case.sm_scale, rows=rows)
