"""The extension configurations the benchmark times, at their full sizes,
against the fp64 oracle: cross attention (4096 queries at the end of 16384
keys), grouped K/V heads (B = 2, H = 32 over 8 K/V heads, N = 8192, forward
and backward), a 4096-key window over N = 32768, and split-KV decoding of
one token per sequence against a 32768-token cache (B = 8, H = 32 over 8
K/V heads).  The kernels and launch shapes are the ones the benchmark runs,
since both pick them from the problem's shape alone.

Every element is checked where the oracle finishes in seconds (the
forwards and decoding); the grouped backward is checked on one whole K/V
head group (its four query heads' dQ and the group's dK, dV), the window
on three whole heads.  Comparison rules: gpu_checks.py.
"""

import math
from types import SimpleNamespace

import numpy as np
import pytest

from gpu_checks import check_decode, check_gradients, empty_rows
from io_aware_tiled_fa_amd.inputs import make_inputs
from parity import TOL_LSE, TOL_O, TOL_O_MEAN, announce, compare, oracle_forward_by_head, to_device, to_numpy_f32

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fa():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from io_aware_tiled_fa_amd import binding

    binding.load_library()
    return binding


def _forward_every_element(fa, inp, causal, window=0):
    import torch

    scale = 1.0 / math.sqrt(inp.d)
    q, k, v = (to_device(getattr(inp, n + "_bits")) for n in ("q", "k", "v"))
    o, lse = fa.forward(q, k, v, causal=causal, scale=scale, window=window)
    torch.cuda.synchronize()
    o_np, lse_np = to_numpy_f32(o), lse.cpu().numpy().astype(np.float64)
    del q, k, v, o, lse
    o_ref, lse_ref = oracle_forward_by_head(inp, scale, causal, window=window)
    e = empty_rows(inp, causal, window)
    assert np.all(o_np[:, e] == 0.0) and np.all(np.isneginf(lse_np[:, :, e]))
    compare("O", o_np[:, ~e], o_ref[:, ~e], TOL_O, TOL_O_MEAN)
    compare("LSE", lse_np[:, :, ~e], lse_ref[:, :, ~e], TOL_LSE, ulp_aware=False)


@pytest.mark.timeout(600)
def test_cross_b1_h32_nq4096_nk16384(fa):
    announce("next: cross attention B=1 H=32 Nq=4096 Nk=16384 d=128 causal (every element)")
    inp = make_inputs(1, 32, 4096, 128, N_k=16384, seed=31)
    _forward_every_element(fa, inp, True)


@pytest.mark.timeout(600)
def test_gqa_forward_b2_h32_hkv8_n8192(fa):
    announce("next: grouped heads forward B=2 H=32 Hkv=8 N=8192 d=128 causal (every element)")
    inp = make_inputs(2, 32, 8192, 128, H_kv=8, seed=32)
    _forward_every_element(fa, inp, True)


@pytest.mark.timeout(600)
def test_gqa_backward_b2_h32_hkv8_n8192(fa):
    """The whole problem on the GPU; batch 1's K/V head 5 group (query heads
    20-23) against the oracle under the gradient error model."""
    import torch

    announce("next: grouped heads backward B=2 H=32 Hkv=8 N=8192 d=128 causal (one K/V head group)")
    inp = make_inputs(2, 32, 8192, 128, H_kv=8, seed=33, with_do=True)
    scale = 1.0 / math.sqrt(128)
    q, k, v, do = (to_device(getattr(inp, n + "_bits")) for n in ("q", "k", "v", "do"))
    o, lse = fa.forward(q, k, v, causal=True, scale=scale)
    dq, dk, dv = fa.backward(q, k, v, o, lse, do, causal=True, scale=scale)
    torch.cuda.synchronize()
    b, hk, G = 1, 5, 4
    hs = slice(hk * G, hk * G + G)
    part = SimpleNamespace(q=inp.q[b:b + 1, :, hs], k=inp.k[b:b + 1, :, hk:hk + 1], v=inp.v[b:b + 1, :, hk:hk + 1],
                           do=inp.do[b:b + 1, :, hs], N=inp.N, N_k=inp.N_k, d=inp.d)
    check_gradients(part, True, scale, 0, o[b:b + 1, :, hs], lse[b:b + 1, hs],
                    (dq[b:b + 1, :, hs], dk[b:b + 1, :, hk:hk + 1], dv[b:b + 1, :, hk:hk + 1]))


@pytest.mark.timeout(600)
def test_window4096_b1_h32_n32768(fa):
    """The whole problem on the GPU; heads 0, 13 and 31 against the oracle."""
    import torch

    announce("next: window 4096 B=1 H=32 N=32768 d=128 causal (three whole heads)")
    inp = make_inputs(1, 32, 32768, 128, seed=34)
    scale, W = 1.0 / math.sqrt(128), 4096
    q, k, v = (to_device(getattr(inp, n + "_bits")) for n in ("q", "k", "v"))
    o, lse = fa.forward(q, k, v, causal=True, scale=scale, window=W)
    torch.cuda.synchronize()
    heads = [0, 13, 31]
    o_np = to_numpy_f32(o[:, :, heads])
    lse_np = lse[:, heads].cpu().numpy().astype(np.float64)
    del q, k, v, o, lse
    part = SimpleNamespace(q=inp.q[:, :, heads], k=inp.k[:, :, heads], v=inp.v[:, :, heads], N=inp.N, N_k=inp.N_k)
    o_ref, lse_ref = oracle_forward_by_head(part, scale, True, window=W)
    compare("O", o_np, o_ref, TOL_O, TOL_O_MEAN)
    compare("LSE", lse_np, lse_ref, TOL_LSE, ulp_aware=False)


@pytest.mark.timeout(600)
def test_decode_b8_h32_hkv8_nk32768(fa):
    announce("next: split-KV decoding B=8 H=32 Hkv=8 Nq=1 Nk=32768 d=128 causal (every element)")
    inp = make_inputs(8, 32, 1, 128, N_k=32768, H_kv=8, seed=35)
    check_decode(fa, inp, True, 1.0 / math.sqrt(128))
