"""Shared GPU-versus-oracle checks for the general entry points (any N_q,
N_k, grouped K/V heads, sliding window), used by the GPU test modules.

Rows that see no key (possible when N_q > N_k under the causal mask, or
with a window) must give exactly O = 0, LSE = -inf and dQ = 0; the other
rows are compared element by element with the fp64 oracle.  O and LSE take
the fixed gates.  The gradients take, per element, the larger of the fixed
gate and the error bound derived from the bfloat16 arithmetic (parity.py):
with few visible keys each probability is large, and the bf16 rounding of
dS then enters every term of a dK sum with weights the long-sequence
workloads never see.
"""

import numpy as np

import oracle
from parity import (TOL_GRAD, TOL_LSE, TOL_O, TOL_O_MEAN, backward_error_bound, compare, to_device,
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
    rq, rk, rv = oracle.attention_backward(inp.q, inp.k, inp.v, inp.do, scale, causal, window=window)
    o_ref, _ = oracle.attention_forward(inp.q, inp.k, inp.v, scale, causal, window=window)
    bounds = backward_error_bound(inp.q, inp.k, inp.v, inp.do, o_ref, scale, causal, window)
    e = empty_rows(inp, causal, window)
    dq_np = to_numpy_f32(dq)
    assert np.all(dq_np[:, e] == 0.0), "rows without a visible key must give dQ = 0"
    for name, got, ref, bound in (("dQ", dq_np, rq, bounds[0]), ("dK", to_numpy_f32(dk), rk, bounds[1]),
                                  ("dV", to_numpy_f32(dv), rv, bounds[2])):
        compare(name, got, ref, TOL_GRAD, bound=np.maximum(bound, TOL_GRAD))
    return dq, dk, dv
