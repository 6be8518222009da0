"""Ragged tiles read zeros past the end of a head, never the memory after it.

The kernels copy whole key tiles (and, in the dK/dV kernel, whole 32-row
query blocks) through buffer resources sized to each head's rows, so that a
tile running past N_k (or N_q) reads zeros.  Here every input tensor sits at
the start of a larger allocation whose remainder is filled with NaN: any
read past a tensor's end (the last batch's last rows) would bring NaN into
the products (masked scores are replaced, but a NaN value row times a zero
probability is still NaN).  Outputs must be finite and match the oracle.
"""

import math

import numpy as np
import pytest

import oracle
from gpu_checks import check_gradients, empty_rows
from io_aware_tiled_fa_amd.inputs import make_inputs
from parity import TOL_LSE, TOL_O, TOL_O_MEAN, announce, compare, to_numpy_f32

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fa():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from io_aware_tiled_fa_amd import binding

    binding.load_library()
    return binding


def poisoned(bits: np.ndarray):
    """The bf16 tensor with these bits at the start of an allocation that
    holds 256 more rows' worth of NaN after it (a contiguous view)."""
    import torch

    shape = bits.shape
    n = int(np.prod(shape))
    pad = 256 * shape[2] * shape[3]
    buf = torch.full((n + pad,), float("nan"), dtype=torch.bfloat16, device="cuda")
    src = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16).reshape(-1)).view(torch.bfloat16)
    buf[:n].copy_(src.to("cuda"))
    return buf[:n].view(shape)


CASES = [
    # B, H, H_kv, N_q, N_k, d, causal, window
    (1, 2, 2, 100, 100, 128, True, 0),
    (1, 2, 2, 100, 100, 64, False, 0),
    (2, 2, 2, 333, 333, 128, False, 0),
    (1, 4, 2, 77, 333, 64, False, 0),
    (1, 2, 2, 300, 130, 128, True, 0),
    (2, 4, 1, 201, 201, 128, True, 50),
    (1, 2, 2, 1, 5, 64, False, 0),
]


@pytest.mark.parametrize("B,H,Hkv,Nq,Nk,d,causal,window", CASES)
def test_ragged_tiles_read_zeros(fa, B, H, Hkv, Nq, Nk, d, causal, window):
    import torch

    announce(f"over-read B={B} H={H} Hkv={Hkv} Nq={Nq} Nk={Nk} d={d} causal={causal} W={window}")
    inp = make_inputs(B, H, Nq, d, N_k=Nk, H_kv=Hkv, seed=8800 + Nq + Nk + d, with_do=True)
    scale = 1.0 / math.sqrt(d)
    q, k, v, do = (poisoned(getattr(inp, n + "_bits")) for n in ("q", "k", "v", "do"))
    o, lse = fa.forward(q, k, v, causal=causal, scale=scale, window=window)
    torch.cuda.synchronize()
    o_np = to_numpy_f32(o)
    assert np.isfinite(o_np).all(), "NaN from past a tensor's end reached O"
    o_ref, lse_ref = oracle.attention_forward(inp.q, inp.k, inp.v, scale, causal, window=window)
    e = empty_rows(inp, causal, window)
    compare("O", o_np[:, ~e], o_ref[:, ~e], TOL_O, TOL_O_MEAN)
    compare("LSE", lse.cpu().numpy()[:, :, ~e], lse_ref[:, :, ~e], TOL_LSE, ulp_aware=False)
    # the backward reads the forward's O from a poisoned allocation as well
    o_p = poisoned(o.view(torch.int16).cpu().numpy().view(np.uint16))
    grads = fa.backward(q, k, v, o_p, lse, do, causal=causal, scale=scale, window=window)
    torch.cuda.synchronize()
    for name, g in zip(("dQ", "dK", "dV"), grads):
        assert np.isfinite(to_numpy_f32(g)).all(), f"NaN from past a tensor's end reached {name}"
    check_gradients(inp, causal, scale, window, o_p, lse, grads)


@pytest.mark.parametrize("Nk", [5, 1000])
def test_decode_ragged_stages_read_zeros(fa, Nk):
    """The split-KV decode kernel copies stages of 128 keys."""
    import torch

    announce(f"over-read decode Nk={Nk}")
    inp = make_inputs(2, 8, 1, 128, N_k=Nk, H_kv=2, seed=8900 + Nk)
    q, k, v = (poisoned(getattr(inp, n + "_bits")) for n in ("q", "k", "v"))
    o, lse = fa.decode(q, k, v, causal=True)
    torch.cuda.synchronize()
    o_np = to_numpy_f32(o)
    assert np.isfinite(o_np).all(), "NaN from past a tensor's end reached O"
    o_ref, lse_ref = oracle.attention_forward(inp.q, inp.k, inp.v, 1.0 / math.sqrt(128), True)
    compare("O", o_np, o_ref, TOL_O, TOL_O_MEAN)
    compare("LSE", lse.cpu().numpy(), lse_ref, TOL_LSE, ulp_aware=False)
