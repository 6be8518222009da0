"""The gradient gate of the GPU tests, checked on the CPU.

The backward tests hold each element of dQ, dK and dV to the error model of
parity.backward_error_model.  Here that model meets an emulation of the
kernels' rounding (kernel_emulation.py) on the kinds of shapes the GPU tests
use: the emulation must pass with room to spare, and the same emulation
with each element of dS moved by a few bfloat16 ulps must fail.  So the gate
is neither looser than a plausible mistake nor tighter than correct bf16
arithmetic.
"""

import numpy as np
import pytest

import oracle
from io_aware_tiled_fa_amd.inputs import make_inputs
from kernel_emulation import backward, forward
from parity import backward_error_model, compare_model

CASES = [
    # B, H, H_kv, N_q, N_k, d, causal, window, scale
    (1, 2, 2, 200, 200, 128, True, 1, None),     # every row sees only itself: exact dQ = dK = 0
    (1, 2, 2, 300, 5, 64, False, 0, None),       # five keys, 300 queries
    (1, 2, 2, 300, 5, 128, True, 0, None),       # cross, causal, rows without keys
    (1, 8, 2, 160, 160, 128, True, 0, None),     # grouped heads
    (1, 2, 2, 260, 260, 64, False, 50, None),    # two-sided window
    (1, 2, 2, 512, 512, 128, True, 0, None),     # long rows
    (1, 2, 2, 192, 192, 128, True, 0, 0.3),      # scale stress cases
    (1, 2, 2, 192, 192, 128, True, 0, -0.3),
    (1, 2, 2, 192, 192, 64, True, 0, 0.0),
]


def _run(B, H, Hkv, Nq, Nk, d, causal, window, scale, ds_ulps=0.0):
    inp = make_inputs(B, H, Nq, d, N_k=Nk, H_kv=Hkv, seed=900 + Nq + Nk + d + window, with_do=True)
    scale = 1.0 / np.sqrt(d) if scale is None else scale
    o, lse = forward(inp.q, inp.k, inp.v, scale, causal, window)
    grads = backward(inp.q, inp.k, inp.v, inp.do, o, lse, scale, causal, window, ds_ulps=ds_ulps)
    ref = oracle.attention_backward(inp.q, inp.k, inp.v, inp.do, scale, causal, window=window)
    det, slack = backward_error_model(inp.q, inp.k, inp.v, inp.do, o, lse, scale, causal, window)
    return grads, ref, det, slack


@pytest.mark.parametrize("case", CASES)
def test_emulated_kernels_pass_the_gate(case):
    grads, ref, det, slack = _run(*case)
    for name, g, r, dt, sl in zip(("dQ", "dK", "dV"), grads, ref, det, slack):
        st = compare_model(name, g, r, dt, sl)
        # the largest element uses well under its limit: the model is not a
        # hair's breadth from failing correct arithmetic
        assert st["max_frac_of_limit"] < 0.8, (name, st)


@pytest.mark.parametrize("case", CASES)
def test_planted_ds_error_fails_the_gate(case):
    """Each dS element moved by 3 bf16 ulps (random directions): dQ or dK
    must fail.  (W = 1 has dS = 0 exactly, where the planted error is 0 too;
    there the exact zero is the check, see test_window_one_is_tight.)"""
    if case[7] == 1:
        pytest.skip("dS is exactly zero with a one-key window")
    if case[8] == 0.0:
        pytest.skip("with scale 0, dQ = dK = 0 whatever dS is")
    grads, ref, det, slack = _run(*case, ds_ulps=3.0)
    failed = []
    for name, g, r, dt, sl in zip(("dQ", "dK"), grads[:2], ref[:2], det[:2], slack[:2]):
        try:
            compare_model(name, g, r, dt, sl)
        except AssertionError:
            failed.append(name)
    assert failed, "a 3-ulp error in every dS element passed the gate"


def test_window_one_is_tight():
    """With a one-key window the exact dQ and dK are 0; the gate allows only
    float32-level noise there (the earlier first-order bound allowed 0.136)."""
    grads, ref, det, slack = _run(*CASES[0])
    assert np.abs(ref[0]).max() < 1e-12 and np.abs(ref[1]).max() < 1e-12
    assert slack[0].max() < 1e-3 and slack[1].max() < 1e-3


def test_planted_scale_error_fails_the_gate():
    """dQ off by a factor 1 + 2^-6 (a wrong scale constant) fails."""
    grads, ref, det, slack = _run(*CASES[5])
    with pytest.raises(AssertionError):
        compare_model("dQ", grads[0] * (1 + 2.0 ** -6), ref[0], det[0], slack[0])
