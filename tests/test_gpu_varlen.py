"""Any sequence length and cross attention (N_q != N_k): fa_fwd_qk and
fa_bwd_qk through the C ABI against the fp64 oracle.

Lengths are chosen to end ragged in every tile size the kernels use (query
blocks of 128 or 256 rows in the forward, 32-row query blocks and 128-key
blocks in the backward, 64-key tiles everywhere), including single rows and
keys.  Under the causal mask the keys are aligned to the end of the query
block (key j is visible to query i iff j <= i + N_k - N_q), so with
N_q > N_k the first N_q - N_k rows see no key: their O and dQ must be exactly
zero and their LSE -inf.

The comparison rules are those of gpu_checks.py.
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


SELF = [
    # B, H, N, d, causal  (square, lengths that are not multiples of any tile)
    (1, 1, 1, 64, False),
    (1, 2, 1, 128, True),
    (2, 3, 37, 64, True),
    (2, 3, 100, 64, False),
    (1, 2, 129, 128, True),
    (1, 2, 129, 128, False),
    (2, 2, 333, 128, True),
    (1, 3, 601, 64, True),
    (1, 2, 1000, 128, False),
]

CROSS = [
    # B, H, N_q, N_k, d, causal
    (1, 2, 64, 512, 128, True),     # queries at the end of a longer context
    (2, 2, 100, 777, 64, True),
    (2, 2, 100, 777, 64, False),
    (1, 3, 600, 161, 128, False),
    (1, 3, 600, 161, 128, True),    # 439 rows see no key
    (1, 2, 300, 5, 64, False),      # one partial key tile
    (1, 2, 300, 5, 128, True),
    (2, 4, 1, 3000, 128, True),     # one query row (decode shape)
    (1, 2, 3, 1, 64, False),
    (1, 2, 257, 1023, 128, True),
]


@pytest.mark.parametrize("B,H,N,d,causal", SELF)
def test_forward_any_length(fa, B, H, N, d, causal):
    announce(f"fwd any-length B={B} H={H} N={N} d={d} causal={causal}")
    inp = make_inputs(B, H, N, d, seed=3000 + N + d)
    check_forward(fa, inp, causal, 1.0 / math.sqrt(d))


@pytest.mark.parametrize("B,H,Nq,Nk,d,causal", CROSS)
def test_forward_cross(fa, B, H, Nq, Nk, d, causal):
    announce(f"fwd cross B={B} H={H} Nq={Nq} Nk={Nk} d={d} causal={causal}")
    inp = make_inputs(B, H, Nq, d, N_k=Nk, seed=4000 + Nq + Nk + d)
    check_forward(fa, inp, causal, 1.0 / math.sqrt(d))


@pytest.mark.parametrize("B,H,N,d,causal", SELF)
def test_backward_any_length(fa, B, H, N, d, causal):
    announce(f"bwd any-length B={B} H={H} N={N} d={d} causal={causal}")
    inp = make_inputs(B, H, N, d, seed=5000 + N + d, with_do=True)
    check_backward(fa, inp, causal, 1.0 / math.sqrt(d))


@pytest.mark.parametrize("B,H,Nq,Nk,d,causal", CROSS)
def test_backward_cross(fa, B, H, Nq, Nk, d, causal):
    announce(f"bwd cross B={B} H={H} Nq={Nq} Nk={Nk} d={d} causal={causal}")
    inp = make_inputs(B, H, Nq, d, N_k=Nk, seed=6000 + Nq + Nk + d, with_do=True)
    check_backward(fa, inp, causal, 1.0 / math.sqrt(d))


@pytest.mark.timeout(600)
@pytest.mark.parametrize("B,H,Nq,Nk,d,causal", [(2, 8, 1100, 1100, 64, True), (1, 16, 900, 1300, 64, False),
                                                 (2, 8, 1500, 1500, 128, True)])
def test_backward_grid_ragged(fa, B, H, Nq, Nk, d, causal):
    """Backward on grids whose (batch, head) count is a multiple of 8, so
    both kernels take the per-XCD head order, over several workgroup rounds
    and ragged in every tile size.  Every element under the error model."""
    announce(f"bwd grid B={B} H={H} Nq={Nq} Nk={Nk} d={d} causal={causal}")
    inp = make_inputs(B, H, Nq, d, N_k=Nk, seed=7000 + Nq + Nk + d, with_do=True)
    check_backward(fa, inp, causal, 1.0 / math.sqrt(d))


def test_cross_equals_suffix_of_self(fa):
    """Causal cross attention of the last N_q queries over N_k keys equals the
    last N_q rows of causal self-attention over all N_k positions, bit for
    bit: both walk the same key tiles with the same mask for those rows.
    Only holds where both launches put the rows in the same tile positions,
    so N_k - N_q is a multiple of the forward's query block."""
    import torch

    announce("fwd cross == suffix of self")
    Nk, Nq, d = 1536, 512, 128
    inp = make_inputs(1, 4, Nk, d, seed=77)
    q, k, v = (to_device(getattr(inp, n + "_bits")) for n in ("q", "k", "v"))
    o_full, lse_full = fa.forward(q, k, v, causal=True)
    o_suf, lse_suf = fa.forward(q[:, Nk - Nq:].contiguous(), k, v, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o_suf.view(torch.int16), o_full[:, Nk - Nq:].view(torch.int16))
    assert torch.equal(lse_suf, lse_full[:, :, Nk - Nq:])


@pytest.mark.timeout(600)
@pytest.mark.parametrize("B,H,Nq,Nk", [(2, 32, 6000, 6000), (4, 32, 3000, 4500)])
def test_forward_large_grid_ragged(fa, B, H, Nq, Nk):
    """Causal d = 128 grids of at least 1024 workgroups of 384 rows run the
    12-wave forward kernel; these end ragged in its 384-row query tiles.
    Every element against the oracle."""
    import torch

    from parity import TOL_LSE, TOL_O, TOL_O_MEAN, compare, oracle_forward_by_head, to_numpy_f32

    announce(f"fwd large grid B={B} H={H} Nq={Nq} Nk={Nk} d=128 causal (every element)")
    inp = make_inputs(B, H, Nq, 128, N_k=Nk, seed=7700 + Nq)
    q, k, v = (to_device(getattr(inp, n + "_bits")) for n in ("q", "k", "v"))
    o, lse = fa.forward(q, k, v, causal=True)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle_forward_by_head(inp, 1.0 / math.sqrt(128), True)
    compare("O", to_numpy_f32(o), o_ref, TOL_O, TOL_O_MEAN)
    compare("LSE", lse.cpu().numpy(), lse_ref, TOL_LSE, ulp_aware=False)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("B,H,Nq,Nk", [(4, 16, 2000, 2000), (4, 16, 1900, 2100)])
def test_forward_d64_large_grid_ragged(fa, B, H, Nq, Nk):
    """Full attention at d = 64 on grids of at least 512 workgroups of 256
    rows runs the 8-wave d = 64 kernel; these end ragged in its 256-row query
    tiles and 64-key tiles.  Every element against the oracle."""
    import torch

    from parity import TOL_LSE, TOL_O, TOL_O_MEAN, compare, oracle_forward_by_head, to_numpy_f32

    announce(f"fwd d=64 large grid B={B} H={H} Nq={Nq} Nk={Nk} full attention (every element)")
    inp = make_inputs(B, H, Nq, 64, N_k=Nk, seed=6400 + Nq)
    q, k, v = (to_device(getattr(inp, n + "_bits")) for n in ("q", "k", "v"))
    o, lse = fa.forward(q, k, v, causal=False)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle_forward_by_head(inp, 1.0 / math.sqrt(64), False)
    compare("O", to_numpy_f32(o), o_ref, TOL_O, TOL_O_MEAN)
    compare("LSE", lse.cpu().numpy(), lse_ref, TOL_LSE, ulp_aware=False)
