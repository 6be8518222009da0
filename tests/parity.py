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
    stats["max_limit"] = float(limit.max()) if err.size else 0.0
    print(f"  {name}: {stats}", flush=True)
    record_stats(name, stats)
    worst = np.unravel_index(np.argmax(err - limit), err.shape) if err.size else None
    assert (err <= limit).all(), (
        f"{name}: {int((err > limit).sum())} elements beyond tolerance; worst at {worst}: "
        f"got {got[worst]:.6g} ref {ref[worst]:.6g} limit {limit[worst]:.3g}")
    if mean_tol is not None:
        assert stats["mean_abs"] <= mean_tol, f"{name}: mean abs {stats['mean_abs']:.3e} > {mean_tol}"
    return stats


def announce(msg: str):
    set_case(msg)
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


def oracle_forward_by_head(inp, scale, causal, window=0, workers=None, row_block=1024):
    """oracle.attention_forward of every (batch, head), the heads spread over
    a thread pool (numpy releases the interpreter lock in its array loops
    and matrix products).  Same layouts and values as one call of the
    oracle on the whole batch; for the long workloads, whose score rows the
    oracle materialises block by block."""
    import os
    from concurrent.futures import ThreadPoolExecutor

    import oracle

    B, n_q, H, d = inp.q.shape
    G = H // inp.k.shape[2]
    if workers is None:
        workers = max(1, min(16, len(os.sched_getaffinity(0))))
    o = np.empty((B, n_q, H, d))
    lse = np.empty((B, H, n_q))
    q, k, v = inp.q, inp.k, inp.v

    def one(bh):
        b, h = divmod(bh, H)
        ob, lb = oracle.attention_forward(q[b:b + 1, :, h:h + 1], k[b:b + 1, :, h // G:h // G + 1],
                                          v[b:b + 1, :, h // G:h // G + 1], scale, causal,
                                          row_block=row_block, window=window)
        o[b, :, h] = ob[0, :, 0]
        lse[b, h] = lb[0, 0]
        return bh

    done = 0
    with ThreadPoolExecutor(max_workers=workers) as ex:
        for _ in ex.map(one, range(B * H)):
            done += 1
            if done % max(1, (B * H) // 8) == 0:
                print(f"  oracle: {done}/{B * H} heads", flush=True)
    return o, lse


# ---------------------------------------------------------------------------
# Error bound of the forward, derived from the arithmetic, for stress cases
# outside the five workloads (for example much larger softmax scales).
# First order in the bfloat16 unit roundoff u = 2^-8 (8 significant bits:
# half an ulp is at most 2^-8 of the value), worst case over signs: P is
# rounded to bf16 for the PV product (relative u each) and the row sum is
# taken from the unrounded P (another u):
#     |O_gpu_ic - O_ic| <= 2u sum_j P_ij |V_jc|
# plus half an ulp of the bf16 output.

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


def forward_error_bound(q, k, v, scale, causal, window=0, workers=1):
    """Per-element bound for O, layout [B, N, H, d] (K, V may have fewer heads);
    the heads spread over ``workers`` threads."""
    from concurrent.futures import ThreadPoolExecutor

    B, N, H, d = q.shape
    G = H // k.shape[2]
    out = np.empty((B, N, H, v.shape[3]))

    def one(bh):
        b, h = divmod(bh, H)
        p = _probabilities(q[b, :, h].astype(np.float64), k[b, :, h // G].astype(np.float64), scale, causal,
                           window)
        out[b, :, h] = 2 * U_BF16 * (p @ np.abs(v[b, :, h // G].astype(np.float64)))

    with ThreadPoolExecutor(max_workers=max(1, workers)) as ex:
        list(ex.map(one, range(B * H)))
    return out


# ---------------------------------------------------------------------------
# Error model of the backward kernels, per element of dQ, dK and dV.
#
# The kernels recompute P from the forward's float32 LSE, form D_i = dO_i . O_i
# from the forward's bfloat16 O, round P (for dV) and dS = P (dP - D) (for dQ
# and dK) to bfloat16 for the matrix cores, and accumulate in float32.  So
#  * a signed error that follows from the forward's O and LSE themselves:
#    with r_i = exp(LSE_i - LSE_gpu_i) and dD_i = dO_i . (O_gpu_i - O_i), the
#    kernels use P_ij r_i and dS_ij = P_ij r_i (dP_ij - D_i - dD_i); its effect
#    on every gradient is computed exactly here from the GPU's O and LSE;
#  * the bfloat16 roundings of P and dS: each a relative error within
#    +-u = 2^-8, modelled as independent and uniform (variance u^2 / 3), so a
#    sum of such terms has a standard deviation sigma (the probabilistic
#    rounding-error analysis of Higham and Mary, SIAM J. Sci. Comput. 2019);
#    LAMBDA sigma is allowed;
#  * float32 arithmetic, worst case: the d-term sums of S, dP and D, exp2 and
#    the scale factor, and the long sums over keys or queries (taken as
#    3 u32 sqrt(n) of the sum of magnitudes);
#  * the final rounding of the output to bfloat16: half an ulp.
# Checked on the CPU against an emulation of the kernels' arithmetic
# (tests/test_gate_model.py): the emulation passes, and a planted error of a
# few bf16 ulps per element of dS fails.

LAMBDA = 6.0
U32 = 2.0 ** -24


def backward_error_model(q, k, v, do, o_gpu, lse_gpu, scale, causal, window=0):
    """(det, slack) per gradient: det[i] is the signed error the GPU's O and
    LSE imply for (dQ, dK, dV)[i], slack[i] what the other roundings may add
    (without the output's half ulp).  Inputs float arrays [B, N, H, d],
    o_gpu the GPU forward's O, lse_gpu its LSE [B, H, N_q]."""
    B, n_q, H, d = q.shape
    n_k, H_kv = k.shape[1], k.shape[2]
    G = H // H_kv
    det = [np.zeros((B, n_q, H, d)), np.zeros((B, n_k, H_kv, d)), np.zeros((B, n_k, H_kv, d))]
    var = [np.zeros_like(x) for x in det]
    f32 = [np.zeros_like(x) for x in det]
    sc = abs(scale)
    for b in range(B):
        for h in range(H):
            hk = h // G
            qh, gh = q[b, :, h].astype(np.float64), do[b, :, h].astype(np.float64)
            kh, vh = k[b, :, hk].astype(np.float64), v[b, :, hk].astype(np.float64)
            og = np.asarray(o_gpu[b, :, h], dtype=np.float64)
            lg = np.asarray(lse_gpu[b, h], dtype=np.float64)
            vis = _visible(n_q, n_k, causal, window)
            s = np.where(vis, scale * (qh @ kh.T), -np.inf)
            m = s.max(axis=1)
            seen = np.isfinite(m)
            m0 = np.where(seen, m, 0.0)
            e = np.exp(s - m0[:, None])
            tot = e.sum(axis=1)
            p = e / np.where(seen, tot, 1.0)[:, None]
            lse = m0 + np.log(np.where(seen, tot, 1.0))
            dp = gh @ vh.T
            dd = (p * dp).sum(axis=1)
            ds = p * (dp - dd[:, None])
            with np.errstate(invalid="ignore", over="ignore"):
                r = np.where(seen, np.exp(lse - np.where(seen, lg, 0.0)), 1.0)
            d_d = (gh * (og - p @ vh)).sum(axis=1)
            e_ds = p * ((r - 1.0)[:, None] * (dp - dd[:, None]) - (r * d_d)[:, None])
            det[0][b, :, h] = scale * (e_ds @ kh)
            det[1][b, :, hk] += scale * (e_ds.T @ qh)
            det[2][b, :, hk] += ((r - 1.0)[:, None] * p).T @ gh
            u2 = U_BF16 ** 2 / 3.0
            var[0][b, :, h] = u2 * scale ** 2 * ((ds * ds) @ (kh * kh))
            var[1][b, :, hk] += u2 * scale ** 2 * ((ds * ds).T @ (qh * qh))
            var[2][b, :, hk] += u2 * ((p * p).T @ (gh * gh))
            s0 = np.where(vis, np.abs(s), 0.0)
            rel_p = U32 * (sc * d * (np.abs(qh) @ np.abs(kh).T) + 2.0 * s0 + 4.0)
            abs_dpd = U32 * d * (np.abs(gh) @ np.abs(vh).T + np.abs(gh * og).sum(axis=1)[:, None])
            err_ds = np.abs(ds) * rel_p + p * abs_dpd
            acc_k = 3.0 * U32 * np.sqrt(n_k)
            acc_q = 3.0 * U32 * np.sqrt(n_q * G)
            f32[0][b, :, h] = sc * (err_ds @ np.abs(kh) + acc_k * (np.abs(ds) @ np.abs(kh)))
            f32[1][b, :, hk] += sc * (err_ds.T @ np.abs(qh) + acc_q * (np.abs(ds).T @ np.abs(qh)))
            f32[2][b, :, hk] += (p * rel_p).T @ np.abs(gh) + acc_q * (p.T @ np.abs(gh))
    slack = [LAMBDA * np.sqrt(vv) + ff for vv, ff in zip(var, f32)]
    return det, slack


def compare_model(name: str, got, ref, det, slack) -> dict:
    """Check |got - ref - det| <= slack + half a bf16 ulp of the output, per
    element; report the raw error against the oracle and the largest
    fraction of its limit any element uses."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, f"{name}: shape {got.shape} vs {ref.shape}"
    assert np.isfinite(got).all(), f"{name}: non-finite values in the GPU result"
    raw = np.abs(got - ref)
    err = np.abs(got - ref - det)
    limit = slack + 0.5 * bf16_ulp(np.maximum(np.abs(ref), np.abs(got))) + 1e-30
    frac = err / limit
    stats = {
        "max_abs": float(raw.max()) if raw.size else 0.0,
        "mean_abs": float(raw.mean()) if raw.size else 0.0,
        "above_raw_tol": int((raw > TOL_GRAD).sum()),
        "max_limit": float(limit.max()) if raw.size else 0.0,
        "max_frac_of_limit": float(frac.max()) if raw.size else 0.0,
        "n": int(raw.size),
    }
    print(f"  {name}: {stats}", flush=True)
    record_stats(name, stats)
    worst = np.unravel_index(np.argmax(frac), err.shape) if err.size else None
    assert (err <= limit).all(), (
        f"{name}: {int((err > limit).sum())} elements beyond the error model; worst at {worst}: "
        f"got {got[worst]:.6g} ref {ref[worst]:.6g} modelled error {det[worst]:.3g} "
        f"limit {limit[worst]:.3g}")
    return stats


# ---------------------------------------------------------------------------
# Per-check statistics, kept for a parity report: when the environment
# variable FA_PARITY_STATS names a file, every check appends one JSON line
# to it (test name, tensor, raw max-abs, mean-abs, count above the raw gate).

_current_case = [""]


def set_case(name: str) -> None:
    _current_case[0] = name


def record_stats(name: str, stats: dict) -> None:
    import json
    import os

    path = os.environ.get("FA_PARITY_STATS")
    if not path:
        return
    with open(path, "a") as f:
        f.write(json.dumps({"case": _current_case[0], "tensor": name, **stats}) + "\n")
