"""Pure-Python brute force of the attention definition (oracle; test
infrastructure). Scalar loops, math.exp and math.fsum, an explicit visibility
test per (token, key); for tiny inputs only. It exists to check the numpy
oracle, not the GPU.
"""
import math


def brute_force(q, k, causal, sigma):
    """q: nested lists [q_b][H][576] of floats, k: [L][576] floats.

    Returns (O [q_b][H][512], LSE [q_b][H]) as nested lists."""
    q_b = len(q)
    L = len(k)
    O, LSE = [], []
    for i in range(q_b):
        pos = L - q_b + i          # global position of query token i
        o_i, lse_i = [], []
        for qh in q[i]:
            vis = [j for j in range(L) if (not causal) or j <= pos]
            if not vis:
                o_i.append([0.0] * 512)
                lse_i.append(-math.inf)
                continue
            s = {j: sigma * math.fsum(a * b for a, b in zip(qh, k[j])) for j in vis}
            m = max(s.values())
            tot = math.fsum(math.exp(s[j] - m) for j in vis)
            lse = m + math.log(tot)
            w = {j: math.exp(s[j] - lse) for j in vis}
            o_i.append([math.fsum(w[j] * k[j][d] for j in vis) for d in range(512)])
            lse_i.append(lse)
        O.append(o_i)
        LSE.append(lse_i)
    return O, LSE
