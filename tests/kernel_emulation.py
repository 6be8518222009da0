"""A float32 emulation of the attention kernels' rounding, for checking the
gradient error model on the CPU (tests/test_gate_model.py).

TEST INFRASTRUCTURE.  It mirrors where the HIP kernels round, not how they
tile: scores and products accumulate in float32, the softmax runs in base 2
from a float32 scale factor, P is rounded to bfloat16 before P V and
P^T dO, dS = P (dP - D) is rounded to bfloat16 before dS K and dS^T Q,
D is formed from the bfloat16 O, and every output is rounded to bfloat16.
It is neither the oracle nor the GPU path: it only has to make errors of
the same kind and size, so that a gate which passes it and fails a planted
mistake is neither too loose nor too tight.
"""

from __future__ import annotations

import numpy as np

from io_aware_tiled_fa_amd.inputs import bf16_bits_from_f32, f32_from_bf16_bits
from parity import _visible

LOG2E = np.float32(1.4426950408889634)
LN2 = np.float32(0.6931471805599453)


def bf16(x) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest even), kept as float32."""
    return f32_from_bf16_bits(bf16_bits_from_f32(np.asarray(x, dtype=np.float32)))


def _scores(qh, kh, scale):
    """Scores in base-2 units, float32: (Q K^T) (scale log2 e)."""
    c = np.float32(abs(scale)) * LOG2E
    sq = -qh if scale < 0 else qh
    return (sq @ kh.T).astype(np.float32) * c


def forward(q, k, v, scale, causal, window=0):
    """O (bf16 values, float32) and LSE (float32) as the forward kernel rounds."""
    B, n_q, H, d = q.shape
    n_k, H_kv = k.shape[1], k.shape[2]
    G = H // H_kv
    o = np.zeros((B, n_q, H, d), dtype=np.float32)
    lse = np.full((B, H, n_q), -np.inf, dtype=np.float32)
    vis = _visible(n_q, n_k, causal, window)
    for b in range(B):
        for h in range(H):
            qh, kh, vh = (x.astype(np.float32) for x in (q[b, :, h], k[b, :, h // G], v[b, :, h // G]))
            t = np.where(vis, _scores(qh, kh, scale), np.float32(-np.inf))
            m = t.max(axis=1)
            seen = np.isfinite(m)
            m0 = np.where(seen, m, np.float32(0))
            p = np.exp2(t - m0[:, None]).astype(np.float32)
            l = p.sum(axis=1, dtype=np.float32)
            acc = (bf16(p) @ vh).astype(np.float32)
            inv = np.where(l > 0, np.float32(1) / np.where(l > 0, l, np.float32(1)), np.float32(0))
            o[b, :, h] = bf16(acc * inv[:, None])
            lse[b, h] = np.where(seen, (m0 + np.log2(np.where(l > 0, l, np.float32(1)))) * LN2, -np.inf)
    return o, lse


def backward(q, k, v, do, o, lse, scale, causal, window=0, ds_ulps=0.0, seed=0):
    """dQ, dK, dV (bf16 values, float32) as the backward kernels round them,
    from the emulated forward's O and LSE.  ``ds_ulps`` plants a mistake: each
    element of dS moves by that many bf16 ulps, in a random direction."""
    B, n_q, H, d = q.shape
    n_k, H_kv = k.shape[1], k.shape[2]
    G = H // H_kv
    rng = np.random.default_rng(seed)
    dq = np.zeros((B, n_q, H, d), dtype=np.float32)
    dk = np.zeros((B, n_k, H_kv, d), dtype=np.float32)
    dv = np.zeros((B, n_k, H_kv, d), dtype=np.float32)
    vis = _visible(n_q, n_k, causal, window)
    c = np.float32(scale) * LOG2E
    for b in range(B):
        for h in range(H):
            hk = h // G
            qh, kh, vh = (x.astype(np.float32) for x in (q[b, :, h], k[b, :, hk], v[b, :, hk]))
            gh, oh = do[b, :, h].astype(np.float32), o[b, :, h].astype(np.float32)
            nl = np.where(np.isfinite(lse[b, h]), -lse[b, h] * LOG2E, np.float32(-np.inf)).astype(np.float32)
            s = (qh @ kh.T).astype(np.float32)
            with np.errstate(invalid="ignore"):
                p = np.exp2(s * c + nl[:, None]).astype(np.float32)
            p = np.where(vis & np.isfinite(nl)[:, None], p, np.float32(0))
            dp = (gh @ vh.T).astype(np.float32)
            dd = (gh * oh).sum(axis=1, dtype=np.float32)
            ds = bf16(p * (dp - dd[:, None]))
            if ds_ulps:
                ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(ds), 2.0 ** -126))) - 7).astype(np.float32)
                ds = (ds + ds_ulps * ulp * rng.choice([-1.0, 1.0], size=ds.shape)).astype(np.float32)
            dq[b, :, h] = bf16(np.float32(scale) * (ds @ kh).astype(np.float32))
            dk[b, :, hk] += np.float32(scale) * (ds.T @ qh).astype(np.float32)
            dv[b, :, hk] += (bf16(p).T @ gh).astype(np.float32)
    return dq, bf16(dk), bf16(dv)
