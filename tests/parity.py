"""Helpers for comparing the HIP path with the fp64 oracle.

Tolerances (fixed by the workloads the kernels are held to):
  O     max-abs <= 1e-2, mean-abs <= 1e-3
  LSE   max-abs <= 1e-3
  dQ, dK, dV max-abs <= 3e-2
O, dQ, dK and dV are bfloat16 outputs: rounding a correct value to bf16 may
by itself move it by half a unit in the last place, which exceeds 1e-2 for
|x| >= 4 (and 3e-2 for |x| >= 8).  So each element is held to
max(tol, one bf16 ulp of the reference); the raw max-abs and the count of
elements above the raw tolerance are reported beside it.  Mean-abs gates
are applied unchanged.
"""

from __future__ import annotations

import sys

import numpy as np

TOL_O = 1e-2
TOL_O_MEAN = 1e-3
TOL_LSE = 1e-3
TOL_GRAD = 3e-2


def bf16_ulp(x: np.ndarray) -> np.ndarray:
    """Spacing of bfloat16 numbers at |x| (8 significant bits)."""
    ax = np.abs(np.asarray(x, dtype=np.float64))
    e = np.floor(np.log2(np.maximum(ax, 2.0 ** -126)))
    return np.exp2(e - 7)


def compare(name: str, got, ref, tol: float, mean_tol: float | None = None,
            ulp_aware: bool = True, bound=None) -> dict:
    """Element-wise check against ``tol`` (ulp-aware, see the module notes);
    with ``bound`` (a per-element error bound from the arithmetic) the limit
    is that bound plus half a bf16 ulp of the reference."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, f"{name}: shape {got.shape} vs {ref.shape}"
    assert np.isfinite(got).all(), f"{name}: non-finite values in the GPU result"
    err = np.abs(got - ref)
    limit = np.maximum(tol, bf16_ulp(ref)) if ulp_aware else np.full(ref.shape, tol)
    if bound is not None:
        limit = np.asarray(bound, dtype=np.float64) + 0.5 * bf16_ulp(ref) + 1e-6
    stats = {
        "max_abs": float(err.max()) if err.size else 0.0,
        "mean_abs": float(err.mean()) if err.size else 0.0,
        "above_raw_tol": int((err > tol).sum()),
        "n": int(err.size),
    }
    print(f"  {name}: {stats}", flush=True)
    worst = np.unravel_index(np.argmax(err - limit), err.shape) if err.size else None
    assert (err <= limit).all(), (
        f"{name}: {int((err > limit).sum())} elements beyond tolerance; worst at {worst}: "
        f"got {got[worst]:.6g} ref {ref[worst]:.6g} limit {limit[worst]:.3g}")
    if mean_tol is not None:
        assert stats["mean_abs"] <= mean_tol, f"{name}: mean abs {stats['mean_abs']:.3e} > {mean_tol}"
    return stats


def announce(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def to_device(bits: np.ndarray, device="cuda"):
    """uint16 bfloat16 bit patterns -> torch bfloat16 tensor on the GPU."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16).to(device)


def to_numpy_f32(t) -> np.ndarray:
    import torch

    return t.detach().to(torch.float32).cpu().numpy()


def sample_rows(n: int, count: int, rng: np.random.Generator, extra=()) -> np.ndarray:
    """Sorted distinct query rows: the first and last rows, tile edges and a
    random sample, plus ``extra``."""
    base = {0, 1, 63, 64, 127, 128, n // 2, n - 65, n - 64, n - 2, n - 1}
    base = {r for r in base if 0 <= r < n}
    base.update(int(r) for r in extra if 0 <= r < n)
    need = max(0, count - len(base))
    pool = np.setdiff1d(np.arange(n), np.array(sorted(base)))
    if need and pool.size:
        base.update(rng.choice(pool, size=min(need, pool.size), replace=False).tolist())
    return np.array(sorted(base), dtype=np.int64)


# ---------------------------------------------------------------------------
# Error bounds derived from the arithmetic, for stress cases outside the five
# workloads (for example much larger softmax scales).  First order in the
# bfloat16 unit roundoff u = 2^-8 (8 significant bits: half an ulp is at
# most 2^-8 of the value), worst case over
# signs:
#   forward: P rounded to bf16 for the PV product (relative u each) and the
#     row sum taken from the unrounded P (another u):
#       |dO_ic| <= 2u sum_j P_ij |V_jc|
#   backward: D_i = dO_i . O_i uses the bf16 O (|dD_i| <= u sum_c |dO_ic O_ic|),
#     dS and P are rounded to bf16 for the products (relative u):
#       |d dS_ij| <= P_ij |dD_i| + u |dS_ij|
#       dQ_ic: |scale| sum_j |d dS_ij| |K_jc|,  dK_jc: |scale| sum_i |d dS_ij| |Q_ic|,
#       dV_jc: u sum_i P_ij |dO_ic|
# Each bound is added to half an ulp of the bf16 output.

U_BF16 = 2.0 ** -8


def _visible(n_q, n_k, causal, window):
    """Keys aligned to the end of the queries; causal and window as in the
    library's conventions (written out here, independent of the oracle)."""
    pos = np.arange(n_q)[:, None] + (n_k - n_q)
    j = np.arange(n_k)[None, :]
    vis = np.ones((n_q, n_k), dtype=bool)
    if causal:
        vis &= j <= pos
    if window > 0:
        vis &= np.abs(pos - j) < window
    return vis


def _probabilities(q, k, scale, causal, window=0):
    """Softmax rows for the bounds; a row that sees no key is all zero."""
    s = scale * (q @ k.T)
    s = np.where(_visible(s.shape[0], s.shape[1], causal, window), s, -np.inf)
    m = s.max(axis=1, keepdims=True)
    m = np.where(np.isfinite(m), m, 0.0)
    e = np.exp(s - m)
    tot = e.sum(axis=1, keepdims=True)
    return e / np.where(tot > 0, tot, 1.0)


def forward_error_bound(q, k, v, scale, causal, window=0):
    """Per-element bound for O, layout [B, N, H, d] (K, V may have fewer heads)."""
    B, N, H, d = q.shape
    G = H // k.shape[2]
    out = np.empty((B, N, H, v.shape[3]))
    for b in range(B):
        for h in range(H):
            p = _probabilities(q[b, :, h].astype(np.float64), k[b, :, h // G].astype(np.float64), scale, causal,
                               window)
            out[b, :, h] = 2 * U_BF16 * (p @ np.abs(v[b, :, h // G].astype(np.float64)))
    return out


def backward_error_bound(q, k, v, do, o_ref, scale, causal, window=0):
    """Per-element bounds for (dQ, dK, dV), layouts like the inputs; a K / V
    head shared by several query heads adds up their bounds."""
    B, N, H, d = q.shape
    n_k, H_kv = k.shape[1], k.shape[2]
    G = H // H_kv
    bq = np.empty((B, N, H, d))
    bk, bv = np.zeros((B, n_k, H_kv, d)), np.zeros((B, n_k, H_kv, d))
    for b in range(B):
        for h in range(H):
            qh, gh = q[b, :, h].astype(np.float64), do[b, :, h].astype(np.float64)
            kh, vh = k[b, :, h // G].astype(np.float64), v[b, :, h // G].astype(np.float64)
            p = _probabilities(qh, kh, scale, causal, window)
            dp = gh @ vh.T
            dd = U_BF16 * np.abs(gh * o_ref[b, :, h]).sum(axis=1, keepdims=True)
            ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
            dds = p * dd + U_BF16 * np.abs(ds)
            bq[b, :, h] = abs(scale) * (dds @ np.abs(kh))
            bk[b, :, h // G] += abs(scale) * (dds.T @ np.abs(qh))
            bv[b, :, h // G] += U_BF16 * (p.T @ np.abs(gh))
    return bq, bk, bv
