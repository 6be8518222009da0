"""The boundary as declared: fa_fwd and fa_bwd called through ctypes with raw
device pointers (no binding in between), against the fp64 oracle.

fa_fwd(q, k, v, o, lse, B, H, N, d, scale, causal, stream) and
fa_bwd(q, k, v, o, lse, dO, dq, dk, dv, B, H, N, d, scale, causal,
workspace, workspace_bytes, stream) are the interface of include/fa.h; the
pages' own interface takes [batch, seq_len, num_heads, head_dim] tensors, a
scale defaulting to 1/sqrt(head_dim) and a causal flag (holysheep.ai review,
"Implementing Flash Attention in Your Architecture").
"""

import math

import pytest

import oracle
from gpu_checks import check_gradients
from io_aware_tiled_fa_amd.inputs import make_inputs
from parity import TOL_LSE, TOL_O, TOL_O_MEAN, announce, compare, to_device, to_numpy_f32

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from io_aware_tiled_fa_amd import binding

    return binding.load_library()


@pytest.mark.parametrize("B,H,N,d,causal", [(2, 3, 200, 128, 1), (1, 4, 130, 64, 0)])
def test_fa_fwd_and_fa_bwd_raw(lib, B, H, N, d, causal):
    import torch

    announce(f"raw C ABI fa_fwd / fa_bwd B={B} H={H} N={N} d={d} causal={causal}")
    inp = make_inputs(B, H, N, d, seed=4242 + N, with_do=True)
    q, k, v, do = (to_device(getattr(inp, n + "_bits")) for n in ("q", "k", "v", "do"))
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    scale = 1.0 / math.sqrt(d)
    stream = torch.cuda.current_stream().cuda_stream
    st = lib.fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                    B, H, N, d, scale, causal, stream)
    assert st == 0, lib.fa_status_string(st)
    ws_bytes = lib.fa_bwd_workspace_size(B, H, N, d)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    st = lib.fa_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), do.data_ptr(),
                    dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, N, d, scale, causal,
                    ws.data_ptr(), ws_bytes, stream)
    assert st == 0, lib.fa_status_string(st)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention_forward(inp.q, inp.k, inp.v, scale, bool(causal))
    compare("O", to_numpy_f32(o), o_ref, TOL_O, TOL_O_MEAN)
    compare("LSE", lse.cpu().numpy(), lse_ref, TOL_LSE, ulp_aware=False)
    check_gradients(inp, bool(causal), scale, 0, o, lse, (dq, dk, dv))
