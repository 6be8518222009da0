"""Brute-force attention with pure-Python loops, for tiny inputs only.

An independent check of the fp64 oracle: every score, exponential and sum is
taken element by element with ``math.fsum`` (exactly rounded sums), so a
mistake in the oracle's array expressions (an index, a transpose, an axis)
cannot hide behind the same mistake here.  Differentiation uses the same
chain rule written per element.
"""

from __future__ import annotations

import math


def _visible(i, j, n_q, n_k, causal, window=0):
    pos = i + (n_k - n_q)  # the query's position among the keys
    if causal and j > pos:
        return False
    if window > 0 and abs(pos - j) >= window:
        return False
    return True


def brute_forward(q, k, v, scale, causal, window=0):
    """q [n_q][d], k [n_k][d], v [n_k][dv] nested lists -> (o, lse)."""
    n_q, n_k = len(q), len(k)
    d, dv = len(q[0]), len(v[0])
    o, lse = [], []
    for i in range(n_q):
        vis = [j for j in range(n_k) if _visible(i, j, n_q, n_k, causal, window)]
        if not vis:
            o.append([0.0] * dv)
            lse.append(-math.inf)
            continue
        s = {j: scale * math.fsum(q[i][c] * k[j][c] for c in range(d)) for j in vis}
        m = max(s.values())
        e = {j: math.exp(s[j] - m) for j in vis}
        total = math.fsum(e.values())
        o.append([math.fsum(e[j] * v[j][c] for j in vis) / total for c in range(dv)])
        lse.append(m + math.log(total))
    return o, lse


def brute_backward(q, k, v, do, scale, causal, window=0):
    """Gradients of sum(O * dO) with respect to q, k, v (nested lists)."""
    n_q, n_k = len(q), len(k)
    d, dv = len(q[0]), len(v[0])
    dq = [[0.0] * d for _ in range(n_q)]
    dk_terms = [[[] for _ in range(d)] for _ in range(n_k)]
    dv_terms = [[[] for _ in range(dv)] for _ in range(n_k)]
    for i in range(n_q):
        vis = [j for j in range(n_k) if _visible(i, j, n_q, n_k, causal, window)]
        if not vis:
            continue
        s = {j: scale * math.fsum(q[i][c] * k[j][c] for c in range(d)) for j in vis}
        m = max(s.values())
        e = {j: math.exp(s[j] - m) for j in vis}
        total = math.fsum(e.values())
        p = {j: e[j] / total for j in vis}
        # dL/dP_ij = dO_i . V_j
        g = {j: math.fsum(do[i][c] * v[j][c] for c in range(dv)) for j in vis}
        pg = math.fsum(p[j] * g[j] for j in vis)
        # dL/dS_ij = P_ij (g_j - sum_l P_il g_l)
        ds = {j: p[j] * (g[j] - pg) for j in vis}
        for c in range(d):
            dq[i][c] = scale * math.fsum(ds[j] * k[j][c] for j in vis)
        for j in vis:
            for c in range(d):
                dk_terms[j][c].append(scale * ds[j] * q[i][c])
            for c in range(dv):
                dv_terms[j][c].append(p[j] * do[i][c])
    dk = [[math.fsum(dk_terms[j][c]) for c in range(d)] for j in range(n_k)]
    dvv = [[math.fsum(dv_terms[j][c]) for c in range(dv)] for j in range(n_k)]
    return dq, dk, dvv
