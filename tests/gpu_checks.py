"""Shared GPU-versus-oracle checks for the general entry points (any N_q,
N_k, grouped K/V heads, sliding window), used by the GPU test modules.

Rows that see no key (possible when N_q > N_k under the causal mask, or
with a window) must give exactly O = 0, LSE = -inf and dQ = 0; the other
rows are compared element by element with the fp64 oracle.  O and LSE take
the fixed gates.  Each gradient element is held to the error model of
parity.backward_error_model: the error the GPU forward's own O and LSE imply
(computed exactly), a statistical allowance for the bfloat16 rounding of P
and dS, float32 terms and the output's half ulp.  The fixed 3e-2 gate would
be far looser than that on these shapes (with few visible keys each
probability is large and every rounding counts fully).
"""

import numpy as np

import oracle
from parity import (TOL_LSE, TOL_O, TOL_O_MEAN, backward_error_model, compare, compare_model, to_device,
                    to_numpy_f32)


def empty_rows(inp, causal, window):
    """Boolean [N_q]: rows with no visible key (from the oracle's mask)."""
    return ~oracle.visible_mask(inp.N, inp.N_k, causal, window=window).any(axis=1)


def check_forward(fa, inp, causal, scale, window=0):
    import torch

    q, k, v = (to_device(getattr(inp, n + "_bits")) for n in ("q", "k", "v"))
    o, lse = fa.forward(q, k, v, causal=causal, scale=scale, window=window)
    torch.cuda.synchronize()
    o_np, lse_np = to_numpy_f32(o), lse.cpu().numpy().astype(np.float64)
    o_ref, lse_ref = oracle.attention_forward(inp.q, inp.k, inp.v, scale, causal, window=window)
    e = empty_rows(inp, causal, window)
    assert np.all(o_np[:, e] == 0.0), "rows without a visible key must give O = 0"
    assert np.all(np.isneginf(lse_np[:, :, e])), "rows without a visible key must give LSE = -inf"
    compare("O", o_np[:, ~e], o_ref[:, ~e], TOL_O, TOL_O_MEAN)
    compare("LSE", lse_np[:, :, ~e], lse_ref[:, :, ~e], TOL_LSE, ulp_aware=False)
    return q, k, v, o, lse


def check_backward(fa, inp, causal, scale, window=0):
    import torch

    q, k, v, o, lse = check_forward(fa, inp, causal, scale, window)
    do = to_device(inp.do_bits)
    dq, dk, dv = fa.backward(q, k, v, o, lse, do, causal=causal, scale=scale, window=window)
    torch.cuda.synchronize()
    check_gradients(inp, causal, scale, window, o, lse, (dq, dk, dv))
    return dq, dk, dv


def check_gradients(inp, causal, scale, window, o, lse, grads):
    """The GPU's (dQ, dK, dV) against the oracle under the error model, given
    the GPU forward's O and LSE that the backward consumed."""
    ref = oracle.attention_backward(inp.q, inp.k, inp.v, inp.do, scale, causal, window=window)
    det, slack = backward_error_model(inp.q, inp.k, inp.v, inp.do, to_numpy_f32(o),
                                      lse.cpu().numpy().astype(np.float64), scale, causal, window)
    e = empty_rows(inp, causal, window)
    got = [to_numpy_f32(t) for t in grads]
    assert np.all(got[0][:, e] == 0.0), "rows without a visible key must give dQ = 0"
    for name, g, r, dt, sl in zip(("dQ", "dK", "dV"), got, ref, det, slack):
        compare_model(name, g, r, dt, sl)


def check_decode(fa, inp, causal, scale, window=0, num_splits=0):
    """Split-KV decoding (fa_fwd_decode) against the oracle, with the
    forward's rules."""
    import torch

    q, k, v = (to_device(getattr(inp, n + "_bits")) for n in ("q", "k", "v"))
    o, lse = fa.decode(q, k, v, causal=causal, scale=scale, window=window, num_splits=num_splits)
    torch.cuda.synchronize()
    o_np, lse_np = to_numpy_f32(o), lse.cpu().numpy().astype(np.float64)
    o_ref, lse_ref = oracle.attention_forward(inp.q, inp.k, inp.v, scale, causal, window=window)
    e = empty_rows(inp, causal, window)
    assert np.all(o_np[:, e] == 0.0), "rows without a visible key must give O = 0"
    assert np.all(np.isneginf(lse_np[:, :, e])), "rows without a visible key must give LSE = -inf"
    compare("O", o_np[:, ~e], o_ref[:, ~e], TOL_O, TOL_O_MEAN)
    compare("LSE", lse_np[:, :, ~e], lse_ref[:, :, ~e], TOL_LSE, ulp_aware=False)
    return o, lse
