"""Split-KV decoding: fa_fwd_decode through the C ABI against the fp64 oracle.

Few query rows (N_q = 1 .. 8) against long key sequences, with grouped K/V
heads packed into one query tile, causal and windowed masks, and the number
of splits chosen by the library or forced (1, a few, more than there are
key stages).  Comparison rules: gpu_checks.py (O and LSE to the fixed
gates, rows without a visible key exactly O = 0 and LSE = -inf).
"""

import math

import pytest

from gpu_checks import check_decode
from io_aware_tiled_fa_amd.inputs import make_inputs
from parity import TOL_LSE, TOL_O, TOL_O_MEAN, announce, compare, to_device, to_numpy_f32

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
    # B, H, H_kv, N_q, N_k, d, causal, window, num_splits
    (2, 8, 2, 1, 5000, 128, True, 0, 0),        # GQA 4:1, ragged last stage
    (1, 32, 8, 4, 8192, 128, True, 0, 0),       # 16 packed rows, 4 positions
    (3, 4, 4, 1, 333, 64, False, 0, 0),         # plain heads, 3 stages
    (1, 16, 2, 1, 10000, 128, True, 1000, 0),   # sliding window
    (1, 8, 1, 3, 2049, 64, False, 300, 0),      # MQA, two-sided window
    (2, 16, 1, 2, 4097, 128, True, 0, 0),       # 32 packed rows
    (1, 4, 1, 8, 5, 128, True, 0, 0),           # N_q > N_k: rows 0..2 see no key
    (1, 8, 2, 1, 7000, 128, True, 0, 1),        # one split: no workspace, direct output
    (1, 8, 2, 1, 7000, 128, True, 0, 3),        # three splits of 19 stages
    (1, 8, 2, 1, 700, 64, True, 0, 1000),       # more splits asked than stages
    (1, 64, 1, 1, 3000, 128, True, 0, 0),       # 64 rows per key head: general forward
]


@pytest.mark.parametrize("B,H,Hkv,Nq,Nk,d,causal,window,splits", CASES)
def test_decode(fa, B, H, Hkv, Nq, Nk, d, causal, window, splits):
    announce(f"decode B={B} H={H} Hkv={Hkv} Nq={Nq} Nk={Nk} d={d} causal={causal} W={window} splits={splits}")
    inp = make_inputs(B, H, Nq, d, N_k=Nk, H_kv=Hkv, seed=9000 + Nq + Nk + window + splits)
    check_decode(fa, inp, causal, 1.0 / math.sqrt(d), window, splits)


@pytest.mark.parametrize("scale", [-0.2, 0.0])
def test_decode_scales(fa, scale):
    announce(f"decode scale={scale}")
    inp = make_inputs(1, 8, 1, 128, N_k=3000, H_kv=2, seed=12)
    check_decode(fa, inp, True, scale)


def test_decode_long_context(fa):
    """A 128K-token cache: 8 query heads over 2 K/V heads, every row checked."""
    announce("decode B=1 H=8 Hkv=2 Nq=1 Nk=131072 d=128 causal")
    inp = make_inputs(1, 8, 1, 128, N_k=131072, H_kv=2, seed=13)
    check_decode(fa, inp, True, 1.0 / math.sqrt(128))


def test_decode_matches_forward(fa):
    """The split path and the general forward agree within the forward gate
    (they sum in different orders, so not bit for bit)."""
    import torch

    announce("decode vs forward")
    inp = make_inputs(2, 16, 2, 128, N_k=6000, H_kv=4, seed=14)
    q, k, v = (to_device(getattr(inp, n + "_bits")) for n in ("q", "k", "v"))
    o1, l1 = fa.decode(q, k, v, causal=True)
    o2, l2 = fa.forward(q, k, v, causal=True)
    torch.cuda.synchronize()
    compare("O", to_numpy_f32(o1), to_numpy_f32(o2), TOL_O, TOL_O_MEAN)
    compare("LSE", l1.cpu().numpy(), l2.cpu().numpy(), TOL_LSE, ulp_aware=False)
