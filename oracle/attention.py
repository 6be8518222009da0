"""Plain fp64 CPU oracle for exact attention, forward and backward.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
baseline leg of the benchmark may import this module.  The HIP library never
calls it, and it shares no code, header, table or helper with the HIP path.

What it computes
----------------
The pages state that FlashAttention returns exactly what standard attention
returns, tiling and the online softmax changing only the order of memory
traffic:

* "Flash Attention Explained: How IO-Aware Computing Made Long Context
  Practical" (institutepm.com), TL;DR and "How Flash Attention Fixes It:
  Tiling and Recomputation" (identical results, the math is identical);
* "What Is Flash Attention? The Real Speed and Memory Gains, Explained"
  (bestllmfor.com), "How Flash Attention works", comparison table (exact, up
  to floating-point rounding);
* "Flash Attention Vs Standard Attention" (avichala.com), "Core Concepts &
  Practical Intuition" (dot products of queries with keys, a softmax, then a
  weighted sum of values).

So this oracle is the plain definition of attention, written out without
tiling: for each (batch, head) it materialises the score matrix S = scale *
Q K^T, masks it when causal, applies the textbook max-shifted softmax along
each row, multiplies by V, and reports the per-row log-sum-exp of the scaled
scores.  The backward differentiates that definition directly (chain rule
through the row softmax), with no use of the forward output O.

Readings where the pages are silent (each also listed in the design notes):

* causal: key j is visible to query i iff j <= i (diagonal included);
  "Flash Attention Vs Standard Attention", "Engineering Perspective" only asks
  that future tokens do not leak.  With N_k != N_q the last query row sees
  every key (keys are aligned to the end of the query block).
* LSE_i = ln(sum_j exp(s_ij)) over visible keys, natural log, s already
  scaled.  The pages do not name it; the backward needs it.
* a row with no visible key (only possible when N_k < N_q under the
  end-aligned causal mask) gives O_i = 0 and LSE_i = -inf.
* inputs are float arrays in [B, N, H, d] layout (the layout of the
  pages' interface, holysheep.ai review, "Implementing Flash Attention in
  Your Architecture"); they are upcast to float64 here.
* grouped-query attention ("Flash Attention Explained", "Flash Attention vs.
  Related Techniques": fewer K/V heads than query heads, orthogonal to the
  method): with H query heads and H_kv key/value heads, query head h reads
  key/value head h // (H / H_kv), so each run of H / H_kv consecutive query
  heads shares one.  The gradient of a shared K/V head is the sum over the
  query heads that read it (chain rule through the sharing).
* sliding window (same section: each token attends only to nearby tokens):
  with window W > 0, key j is visible to query i only if |i' - j| < W,
  i' = i + (N_k - N_q) the query's position among the keys; with the causal
  mask as well that is the W keys i' - W + 1 .. i'.  W = 0 means no window.

Layouts: q [B, N_q, H, d], k and v [B, N_k, H_kv, d], do [B, N_q, H, d].
Outputs: o [B, N_q, H, d], lse [B, H, N_q], dq/dk/dv like q/k/v.  All float64.
"""

from __future__ import annotations

from typing import Optional, Sequence

import numpy as np

__all__ = [
    "visible_mask",
    "scaled_scores",
    "row_softmax",
    "attention_forward",
    "attention_backward",
    "head_forward",
    "head_backward",
    "kv_head",
]


def visible_mask(n_q: int, n_k: int, causal: bool,
                 rows: Optional[np.ndarray] = None, window: int = 0) -> np.ndarray:
    """Boolean [len(rows), n_k]: True where query i may attend to key j.

    Non-causal: every key is visible.  Causal: key j is visible to query i
    iff j <= i + (n_k - n_q) (future tokens masked; "Flash Attention Vs
    Standard Attention", "Engineering Perspective").  A window W > 0 also
    requires |i + (n_k - n_q) - j| < W ("Flash Attention Explained", "Flash
    Attention vs. Related Techniques", sliding window attention).
    """
    if rows is None:
        rows = np.arange(n_q)
    rows = np.asarray(rows, dtype=np.int64)
    pos = rows[:, None] + (n_k - n_q)  # the query's position among the keys
    j = np.arange(n_k, dtype=np.int64)[None, :]
    vis = np.ones((rows.shape[0], n_k), dtype=bool)
    if causal:
        vis &= j <= pos
    if window > 0:
        vis &= np.abs(pos - j) < window
    return vis


def scaled_scores(q: np.ndarray, k: np.ndarray, scale: float) -> np.ndarray:
    """S = scale * Q K^T for one head: q [n, d], k [m, d] -> [n, m], fp64."""
    return float(scale) * (q @ k.T)


def row_softmax(s: np.ndarray, visible: np.ndarray):
    """Max-shifted softmax of each row over its visible entries.

    Returns (P, m, l) with m_i = max visible s_ij, l_i = sum_j exp(s_ij - m_i)
    and P_ij = exp(s_ij - m_i) / l_i (0 where masked).  Rows with nothing
    visible get P = 0, m = -inf, l = 0.
    """
    s = np.where(visible, s, -np.inf)
    m = s.max(axis=1)
    any_visible = np.isfinite(m)
    m_safe = np.where(any_visible, m, 0.0)
    e = np.exp(s - m_safe[:, None])  # masked entries: exp(-inf) = 0
    l = e.sum(axis=1)
    l_safe = np.where(any_visible, l, 1.0)
    p = e / l_safe[:, None]
    return p, m, l


def head_forward(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
                 causal: bool, rows: Optional[np.ndarray] = None, window: int = 0):
    """Attention for one (batch, head): returns (o [n, d], lse [n]).

    ``rows`` restricts the computation to those query positions (each query
    row of attention depends on no other query row, so a subset is exact).
    """
    n_q, n_k = q.shape[0], k.shape[0]
    if rows is None:
        rows = np.arange(n_q)
    q = np.asarray(q[rows], dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    s = scaled_scores(q, k, scale)
    p, m, l = row_softmax(s, visible_mask(n_q, n_k, causal, rows, window))
    o = p @ v
    with np.errstate(divide="ignore"):
        lse = np.where(np.isfinite(m), m + np.log(np.where(l > 0, l, 1.0)), -np.inf)
    return o, lse


def kv_head(h: int, n_heads: int, n_kv_heads: int) -> int:
    """The key/value head that query head h reads (grouped-query attention:
    runs of n_heads // n_kv_heads consecutive query heads share one)."""
    if n_kv_heads <= 0 or n_heads % n_kv_heads:
        raise ValueError(f"{n_heads} query heads cannot share {n_kv_heads} key/value heads evenly")
    return h // (n_heads // n_kv_heads)


def attention_forward(q: np.ndarray, k: np.ndarray, v: np.ndarray,
                      scale: float, causal: bool,
                      rows: Optional[Sequence[int]] = None,
                      row_block: int = 2048, window: int = 0):
    """O = softmax(scale * Q K^T [masked]) V and the per-row LSE, all heads.

    q [B, N_q, H, d]; k, v [B, N_k, H_kv, d].  With ``rows`` only those query
    positions are computed (for every batch and head).  Query rows are
    processed ``row_block`` at a time so a long sequence never needs its
    whole N_q x N_k score matrix at once; rows do not interact, so this
    changes nothing in any row's arithmetic.
    """
    B, n_q, H, d = q.shape
    H_kv = k.shape[2]
    rows = np.arange(n_q) if rows is None else np.asarray(rows, dtype=np.int64)
    o = np.empty((B, rows.shape[0], H, v.shape[3]), dtype=np.float64)
    lse = np.empty((B, H, rows.shape[0]), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            hk = kv_head(h, H, H_kv)
            kh = np.asarray(k[b, :, hk, :], dtype=np.float64)
            vh = np.asarray(v[b, :, hk, :], dtype=np.float64)
            qh = q[b, :, h, :]
            for start in range(0, rows.shape[0], row_block):
                sel = rows[start:start + row_block]
                o_blk, lse_blk = head_forward(qh, kh, vh, scale, causal, sel, window)
                o[b, start:start + sel.shape[0], h, :] = o_blk
                lse[b, h, start:start + sel.shape[0]] = lse_blk
    return o, lse


def head_backward(q: np.ndarray, k: np.ndarray, v: np.ndarray, do: np.ndarray,
                  scale: float, causal: bool, window: int = 0):
    """Gradients of sum(O * dO) for one head by direct differentiation.

    With S = scale Q K^T, P = rowsoftmax(S), O = P V:
      dV = P^T dO
      dP = dO V^T
      dS_i = P_i * (dP_i - sum_j P_ij dP_ij)   (row Jacobian diag(p) - p p^T)
      dQ = scale * dS K
      dK = scale * dS^T Q
    The softmax Jacobian is applied in the form above, from P and dP alone;
    nothing here uses the forward output O.  Recomputing P from Q, K, V
    rather than keeping it follows "Flash Attention Explained", "Recompute
    during backward pass" (institutepm.com); the oracle does it the plain way.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    s = scaled_scores(q, k, scale)
    p, _, _ = row_softmax(s, visible_mask(q.shape[0], k.shape[0], causal, None, window))
    dv = p.T @ do
    dp = do @ v.T
    ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
    dq = float(scale) * (ds @ k)
    dk = float(scale) * (ds.T @ q)
    return dq, dk, dv


def attention_backward(q: np.ndarray, k: np.ndarray, v: np.ndarray,
                       do: np.ndarray, scale: float, causal: bool, window: int = 0):
    """dQ, dK, dV for all heads; same layouts as the inputs, float64.  A
    key/value head shared by several query heads gets the sum of their
    gradients."""
    B, n_q, H, d = q.shape
    n_k, H_kv = k.shape[1], k.shape[2]
    dq = np.empty((B, n_q, H, d), dtype=np.float64)
    dk = np.zeros((B, n_k, H_kv, d), dtype=np.float64)
    dv = np.zeros((B, n_k, H_kv, v.shape[3]), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            hk = kv_head(h, H, H_kv)
            gq, gk, gv = head_backward(q[b, :, h, :], k[b, :, hk, :], v[b, :, hk, :],
                                       do[b, :, h, :], scale, causal, window)
            dq[b, :, h, :] = gq
            dk[b, :, hk, :] += gk
            dv[b, :, hk, :] += gv
    return dq, dk, dv
