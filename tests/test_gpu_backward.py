"""Backward parity: fa_bwd through the C ABI against the fp64 oracle's
direct differentiation.  The GPU backward consumes the GPU forward's O and
LSE; the oracle recomputes everything from Q, K, V and dO in fp64."""

import math

import pytest

import oracle
from io_aware_tiled_fa_amd.inputs import make_inputs, make_workload
from gpu_checks import check_gradients
from parity import TOL_GRAD, announce, compare, to_device, to_numpy_f32

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fa():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from io_aware_tiled_fa_amd import binding

    binding.load_library()
    return binding


def run_bwd(fa, inp, causal, scale):
    import torch

    q, k, v, do = (to_device(getattr(inp, n + "_bits")) for n in ("q", "k", "v", "do"))
    o, lse = fa.forward(q, k, v, causal=causal, scale=scale)
    dq, dk, dv = fa.backward(q, k, v, o, lse, do, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return (dq, dk, dv), (o, lse)


def check_bwd(fa, inp, causal, scale):
    """Small shapes and stress scales: every element under the error model
    of parity.backward_error_model."""
    grads, (o, lse) = run_bwd(fa, inp, causal, scale)
    check_gradients(inp, causal, scale, 0, o, lse, grads)


def check_bwd_workload(fa, inp, causal, scale):
    """A workload: every element against the fixed 3e-2 gate (ulp-aware)."""
    (dq, dk, dv), _ = run_bwd(fa, inp, causal, scale)
    rq, rk, rv = oracle.attention_backward(inp.q, inp.k, inp.v, inp.do, scale, causal)
    compare("dQ", to_numpy_f32(dq), rq, TOL_GRAD)
    compare("dK", to_numpy_f32(dk), rk, TOL_GRAD)
    compare("dV", to_numpy_f32(dv), rv, TOL_GRAD)


SMALL = [
    # B, H, N, d, causal  (N = 192 / 320: the last 128-key block is half full)
    (1, 1, 64, 128, True),
    (1, 2, 192, 128, True),
    (1, 2, 192, 128, False),
    (2, 3, 256, 64, True),
    (2, 3, 256, 64, False),
    (2, 4, 320, 128, True),
    (1, 8, 512, 128, False),
]


@pytest.mark.parametrize("B,H,N,d,causal", SMALL)
def test_backward_small(fa, B, H, N, d, causal):
    announce(f"bwd small B={B} H={H} N={N} d={d} causal={causal}")
    inp = make_inputs(B, H, N, d, seed=2000 + N + d, with_do=True)
    check_bwd(fa, inp, causal, 1.0 / math.sqrt(d))


@pytest.mark.parametrize("scale", [-0.3, 0.3, 0.0])
def test_backward_scales(fa, scale):
    """Negative, larger and zero scales under the same error model."""
    announce(f"bwd scale={scale}")
    inp = make_inputs(1, 2, 256, 128, seed=11, with_do=True)
    check_bwd(fa, inp, True, scale)


@pytest.mark.parametrize("d", [64, 128])
def test_backward_deterministic(fa, d):
    """Each gradient element is summed in a fixed order (no atomics), so two
    runs on the same inputs agree bit for bit."""
    import torch

    announce(f"bwd determinism d={d}")
    inp = make_inputs(2, 4, 384, d, seed=5, with_do=True)
    first, _ = run_bwd(fa, inp, True, 1.0 / math.sqrt(d))
    second, _ = run_bwd(fa, inp, True, 1.0 / math.sqrt(d))
    for name, x, y in zip(("dQ", "dK", "dV"), first, second):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16)), f"{name} differs between runs"


def test_workload_bwd_b4_h16_n4096_d128_causal(fa):
    announce("bwd workload B=4 H=16 N=4096 d=128 causal (every element)")
    inp = make_workload("bwd_b4_h16_n4096_d128_causal")
    check_bwd_workload(fa, inp, True, 1.0 / math.sqrt(128))
