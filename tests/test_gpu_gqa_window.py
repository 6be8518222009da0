"""Grouped-query attention (H_kv < H key/value heads) and sliding windows:
fa_fwd_ex and fa_bwd_ex through the C ABI against the fp64 oracle.

Query head h reads key/value head h // (H / H_kv); the backward sums the
gradients of every query head that reads a key/value head.  A window W keeps
only keys within distance W - 1 of the query's position (before it, and
after it when not causal).  Lengths and windows end ragged in every tile
size the kernels use.  Comparison rules: gpu_checks.py.
"""

import math

import pytest

from gpu_checks import check_backward, check_forward
from io_aware_tiled_fa_amd.inputs import make_inputs
from parity import announce, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fa():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from io_aware_tiled_fa_amd import binding

    binding.load_library()
    return binding


CASES = [
    # B, H, H_kv, N_q, N_k, d, causal, window
    (2, 8, 2, 300, 300, 128, True, 0),      # GQA, 4 query heads per K/V head
    (1, 8, 1, 257, 257, 64, False, 0),      # multi-query attention
    (2, 6, 3, 100, 333, 128, True, 0),      # GQA with cross attention
    (1, 4, 2, 513, 200, 64, True, 0),       # GQA with rows that see no key
    (1, 4, 4, 1000, 1000, 128, True, 128),  # window of one key tile
    (1, 2, 2, 700, 700, 128, True, 1),      # every row sees only itself
    (1, 3, 3, 650, 650, 64, True, 100),     # window not a tile multiple
    (1, 2, 2, 600, 600, 128, False, 300),   # two-sided window
    (1, 2, 2, 200, 900, 128, True, 256),    # window with cross attention
    (1, 2, 2, 500, 120, 64, False, 50),     # two-sided window; the first 331 rows see no key
    (2, 8, 2, 777, 777, 128, True, 200),    # GQA and a window together
    (1, 4, 1, 1, 3000, 128, True, 1000),    # one query row (decode shape), MQA, window
]


def _inputs(B, H, Hkv, Nq, Nk, d, seed, with_do):
    return make_inputs(B, H, Nq, d, N_k=Nk, H_kv=Hkv, seed=seed, with_do=with_do)


@pytest.mark.parametrize("B,H,Hkv,Nq,Nk,d,causal,window", CASES)
def test_forward_gqa_window(fa, B, H, Hkv, Nq, Nk, d, causal, window):
    announce(f"fwd gqa/window B={B} H={H} Hkv={Hkv} Nq={Nq} Nk={Nk} d={d} causal={causal} W={window}")
    inp = _inputs(B, H, Hkv, Nq, Nk, d, 7000 + Nq + Nk + window, False)
    check_forward(fa, inp, causal, 1.0 / math.sqrt(d), window)


@pytest.mark.parametrize("B,H,Hkv,Nq,Nk,d,causal,window", CASES)
def test_backward_gqa_window(fa, B, H, Hkv, Nq, Nk, d, causal, window):
    announce(f"bwd gqa/window B={B} H={H} Hkv={Hkv} Nq={Nq} Nk={Nk} d={d} causal={causal} W={window}")
    inp = _inputs(B, H, Hkv, Nq, Nk, d, 8000 + Nq + Nk + window, True)
    check_backward(fa, inp, causal, 1.0 / math.sqrt(d), window)


@pytest.mark.parametrize("causal", [True, False])
def test_wide_window_equals_no_window(fa, causal):
    """A window wider than every query-key distance must change nothing, bit
    for bit: the kernels walk the same tiles in the same order and the
    window's extra mask never removes a key."""
    import torch

    announce(f"fwd/bwd wide window == no window causal={causal}")
    inp = _inputs(1, 4, 2, 333, 333, 128, 91, True)
    q, k, v, do = (to_device(getattr(inp, n + "_bits")) for n in ("q", "k", "v", "do"))
    o0, l0 = fa.forward(q, k, v, causal=causal)
    o1, l1 = fa.forward(q, k, v, causal=causal, window=10 ** 6)
    g0 = fa.backward(q, k, v, o0, l0, do, causal=causal)
    g1 = fa.backward(q, k, v, o1, l1, do, causal=causal, window=10 ** 6)
    torch.cuda.synchronize()
    assert torch.equal(o0.view(torch.int16), o1.view(torch.int16))
    assert torch.equal(l0, l1)
    for x, y in zip(g0, g1):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))


def test_gqa_equals_repeated_heads(fa):
    """Grouped heads give exactly what plain multi-head attention gives on
    K and V with each head repeated over its group (the same tiles in the
    same order), and dK / dV of a shared head are the group sums of the
    repeated heads' gradients: the group sum is formed once in float32 and
    rounded, the repeated heads' gradients are each rounded first, so the
    two may differ by half a bf16 ulp of every term and of the sum."""
    import torch

    announce("gqa == repeated heads")
    B, H, Hkv, N, d = 2, 8, 2, 384, 128
    inp = _inputs(B, H, Hkv, N, N, d, 92, True)
    q, k, v, do = (to_device(getattr(inp, n + "_bits")) for n in ("q", "k", "v", "do"))
    kr = k.repeat_interleave(H // Hkv, dim=2).contiguous()
    vr = v.repeat_interleave(H // Hkv, dim=2).contiguous()
    o, lse = fa.forward(q, k, v, causal=True)
    o_r, lse_r = fa.forward(q, kr, vr, causal=True)
    dq, dk, dv = fa.backward(q, k, v, o, lse, do, causal=True)
    dq_r, dk_r, dv_r = fa.backward(q, kr, vr, o_r, lse_r, do, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), o_r.view(torch.int16))
    assert torch.equal(lse, lse_r)
    assert torch.equal(dq.view(torch.int16), dq_r.view(torch.int16))
    def half_ulp(x):
        return torch.exp2(torch.floor(torch.log2(x.abs().clamp_min(2.0 ** -126))) - 8)

    for name, got, rep in (("dK", dk, dk_r), ("dV", dv, dv_r)):
        terms = rep.float().view(B, N, Hkv, H // Hkv, d)
        want = terms.sum(dim=3)
        err = (got.float() - want).abs()
        # each term's rounding, the sum's rounding, and the float32 sum itself
        limit = half_ulp(terms).sum(dim=3) + half_ulp(got.float()) + 1e-5 * terms.abs().sum(dim=3)
        assert bool((err <= limit).all()), f"{name}: {(err - limit).max().item()} over the limit"


@pytest.mark.timeout(600)
@pytest.mark.parametrize("causal,window", [(True, 1000), (False, 700)])
def test_window_large_grid_ragged(fa, causal, window):
    """d = 128 windowed grids of at least 1024 workgroups of 384 rows run the
    12-wave forward kernel; N = 6000 ends ragged in its query tiles.  Every
    element against the oracle."""
    import torch

    from parity import TOL_LSE, TOL_O, TOL_O_MEAN, compare, oracle_forward_by_head, to_numpy_f32

    N = 6000
    announce(f"fwd window large grid B=2 H=32 N={N} d=128 causal={causal} W={window} (every element)")
    inp = _inputs(2, 32, 8, N, N, 128, 9100 + window, False)
    q, k, v = (to_device(getattr(inp, n + "_bits")) for n in ("q", "k", "v"))
    o, lse = fa.forward(q, k, v, causal=causal, window=window)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle_forward_by_head(inp, 1.0 / math.sqrt(128), causal, window=window)
    compare("O", to_numpy_f32(o), o_ref, TOL_O, TOL_O_MEAN)
    compare("LSE", lse.cpu().numpy(), lse_ref, TOL_LSE, ulp_aware=False)
