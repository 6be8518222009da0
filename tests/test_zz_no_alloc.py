"""fa_bwd_noalloc: the backward with the row terms in the library's static
scratch instead of a caller's workspace, called through the C ABI, must
give exactly what fa_bwd_ex gives (the same kernels on the same inputs), on
two calls in a row, the second on a smaller problem; and it refuses
problems beyond its scratch before launching anything."""

import math

import pytest

from io_aware_tiled_fa_amd.inputs import make_inputs
from parity import announce, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from io_aware_tiled_fa_amd import binding

    return binding.load_library()


def _both(lib, B, H, Hkv, Nq, Nk, d, causal, window, seed):
    import torch

    inp = make_inputs(B, H, Nq, d, N_k=Nk, H_kv=Hkv, seed=seed, with_do=True)
    q, k, v, do = (to_device(getattr(inp, n + "_bits")) for n in ("q", "k", "v", "do"))
    from io_aware_tiled_fa_amd import binding

    o, lse = binding.forward(q, k, v, causal=causal, window=window)
    scale = 1.0 / math.sqrt(d)
    stream = torch.cuda.current_stream().cuda_stream
    ins = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), do.data_ptr())
    ref = [torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)]
    ws_bytes = lib.fa_bwd_workspace_size(B, H, Nq, d)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
    st = lib.fa_bwd_ex(*ins, *(t.data_ptr() for t in ref), B, H, Hkv, Nq, Nk, d, scale, int(causal), window,
                       ws.data_ptr(), ws_bytes, stream)
    assert st == 0, lib.fa_status_string(st)
    got = [torch.full_like(q, float("nan")), torch.full_like(k, float("nan")), torch.full_like(v, float("nan"))]
    st = lib.fa_bwd_noalloc(*ins, *(t.data_ptr() for t in got), B, H, Hkv, Nq, Nk, d, scale, int(causal), window,
                            stream)
    assert st == 0, lib.fa_status_string(st)
    torch.cuda.synchronize()
    for name, x, y in zip(("dQ", "dK", "dV"), got, ref):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16)), f"{name} differs from fa_bwd_ex"


def test_noalloc_matches_workspace_entry_point(lib):
    """Two calls in a row, the second smaller: the scratch keeps the first
    call's row terms, which the second must not read."""
    announce("fa_bwd_noalloc == fa_bwd_ex, then a smaller problem")
    _both(lib, 2, 8, 2, 1000, 1000, 128, True, 0, 31)
    _both(lib, 1, 2, 2, 300, 77, 64, False, 0, 32)


def test_noalloc_largest_problem(lib):
    """At the limit: B H N_q = 2^21 query rows fill the 16 MiB scratch."""
    announce("fa_bwd_noalloc at 2^21 rows")
    _both(lib, 1, 64, 8, 32768, 2048, 64, True, 0, 33)


def test_noalloc_refuses_more_than_its_scratch(lib):
    """One more row than the scratch holds: FA_ERR_SCRATCH, nothing launched
    (the pointers are never dereferenced)."""
    P = [0x100000000 * (i + 1) for i in range(10)]  # 4 GiB apart: nothing overlaps
    # B = 2049, H = 1, N_q = 1024: 2^21 + 1024 rows, every other size legal
    st = lib.fa_bwd_noalloc(*P[:9], 2049, 1, 1, 1024, 64, 64, 0.125, 1, 0, None)
    assert st == -10
    st = lib.fa_bwd_noalloc(*P[:9], 2048, 1, 1, 1024, 64, 64, float("nan"), 1, 0, None)
    assert st == -7  # 2^21 rows fit: the next check (the scale) refuses it
    assert b"2^21" in lib.fa_status_string(-10)
