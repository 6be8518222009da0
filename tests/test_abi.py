"""The C-ABI library on the CPU: it loads, exports every entry point the
header declares, and rejects bad arguments before touching the GPU.

Every call below carries at least one invalid argument, so validation
returns before any HIP call; the pointer values are never dereferenced.
"""

import math
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")


@pytest.fixture(scope="module")
def lib():
    from io_aware_tiled_fa_amd import binding

    if not os.path.exists(binding.LIB_PATH):
        pytest.skip("libfa.so not built")
    return binding.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    assert declared_functions() == sorted(
        ["fa_fwd", "fa_fwd_qk", "fa_fwd_ex", "fa_fwd_decode", "fa_decode_workspace_size", "fa_bwd",
         "fa_bwd_qk", "fa_bwd_ex", "fa_bwd_noalloc", "fa_bwd_workspace_size", "fa_status_string", "fa_version"])


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings(lib):
    for code in range(0, -11, -1):
        s = lib.fa_status_string(code)
        assert s and s != b"unknown status", code
    assert lib.fa_status_string(-99) == b"unknown status"
    assert lib.fa_version() >= 100


# fake, 256-byte aligned device addresses, far apart so nothing overlaps
P = [0x10000000 * (i + 1) for i in range(12)]


def fwd(lib, q=P[0], k=P[1], v=P[2], o=P[3], lse=P[4], B=1, H=1, N=128, d=64,
        scale=0.125, causal=0):
    return lib.fa_fwd(q, k, v, o, lse, B, H, N, d, scale, causal, None)


def test_fwd_validation(lib):
    assert fwd(lib, q=None) == -1
    assert fwd(lib, lse=None) == -1
    assert fwd(lib, d=96, scale=float("nan")) == -3
    assert fwd(lib, B=0, scale=float("nan")) == -2
    assert fwd(lib, H=-1, scale=float("nan")) == -2
    assert fwd(lib, B=2 ** 20, H=64, N=2 ** 16, d=128) == -2   # > 2^31 elements
    # any sequence length is accepted: the shape passes, the scale is refused
    assert fwd(lib, N=100, scale=float("nan")) == -7
    assert fwd(lib, N=1, scale=float("nan")) == -7
    assert fwd(lib, q=P[0] + 8, scale=float("nan")) == -5
    assert fwd(lib, lse=P[4] + 4, scale=float("nan")) == -5
    assert fwd(lib, scale=float("nan")) == -7
    assert fwd(lib, scale=float("inf")) == -7
    assert fwd(lib, scale=-math.inf) == -7
    assert fwd(lib, causal=2) == -9
    assert fwd(lib, o=P[0]) == -9                    # output aliases Q
    assert fwd(lib, lse=P[2] + 256) == -9            # LSE inside V


def bwd(lib, B=1, H=1, N=128, d=64, ws=P[9], ws_bytes=None, scale=0.125, causal=1, **ptrs):
    p = dict(q=P[0], k=P[1], v=P[2], o=P[3], lse=P[4], do=P[5], dq=P[6], dk=P[7], dv=P[8])
    p.update(ptrs)
    if ws_bytes is None:
        ws_bytes = lib.fa_bwd_workspace_size(B, H, N, d)
    return lib.fa_bwd(p["q"], p["k"], p["v"], p["o"], p["lse"], p["do"], p["dq"], p["dk"], p["dv"],
                      B, H, N, d, scale, causal, ws, ws_bytes, None)


def test_bwd_validation(lib):
    assert bwd(lib, do=None) == -1
    assert bwd(lib, dv=None) == -1
    assert bwd(lib, d=32) == -3
    assert bwd(lib, N=0) == -2
    assert bwd(lib, N=65, scale=float("nan")) == -7   # ragged length passes the shape checks
    assert bwd(lib, dk=P[7] + 2) == -5
    assert bwd(lib, ws=None) == -6
    assert bwd(lib, ws_bytes=1023) == -6               # one byte short of the 1024 needed
    assert bwd(lib, ws=P[9] + 16) == -6               # workspace must be 256-byte aligned
    assert bwd(lib, scale=float("nan")) == -7
    assert bwd(lib, causal=-1) == -9
    assert bwd(lib, dq=P[1]) == -9                    # dQ aliases K
    assert bwd(lib, dk=P[6]) == -9                    # dK aliases dQ
    assert bwd(lib, ws=P[8]) == -9                    # workspace aliases dV


def fwd_qk(lib, Nq=128, Nk=128, B=1, H=1, d=64, scale=0.125, causal=1, **ptrs):
    p = dict(q=P[0], k=P[1], v=P[2], o=P[3], lse=P[4])
    p.update(ptrs)
    return lib.fa_fwd_qk(p["q"], p["k"], p["v"], p["o"], p["lse"], B, H, Nq, Nk, d, scale, causal, None)


def bwd_qk(lib, Nq=128, Nk=128, B=1, H=1, d=64, scale=0.125, causal=1, ws=P[9], ws_bytes=None, **ptrs):
    p = dict(q=P[0], k=P[1], v=P[2], o=P[3], lse=P[4], do=P[5], dq=P[6], dk=P[7], dv=P[8])
    p.update(ptrs)
    if ws_bytes is None:
        ws_bytes = lib.fa_bwd_workspace_size(B, H, Nq, d)
    return lib.fa_bwd_qk(p["q"], p["k"], p["v"], p["o"], p["lse"], p["do"], p["dq"], p["dk"], p["dv"],
                         B, H, Nq, Nk, d, scale, causal, ws, ws_bytes, None)


def test_cross_shape_validation(lib):
    assert fwd_qk(lib, Nq=0) == -2
    assert fwd_qk(lib, Nk=0) == -2
    assert fwd_qk(lib, Nk=-5) == -2
    assert fwd_qk(lib, Nq=1, Nk=2 ** 31 - 1, H=2, d=128) == -2   # K holds > 2^31 elements
    assert fwd_qk(lib, Nq=77, Nk=300, scale=float("nan")) == -7
    # the tile copies address up to 128 rows past a head's last row in 32-bit
    # byte offsets: (N_k + 128) H d must stay under 2^31 as well
    assert fwd_qk(lib, Nq=1, Nk=2 ** 24 - 64, d=128) == -2           # K itself fits, the margin does not
    assert fwd_qk(lib, Nq=1, Nk=2 ** 24 - 128, d=128) == -2
    assert fwd_qk(lib, Nq=1, Nk=2 ** 24 - 129, d=128, scale=float("nan")) == -7
    assert fwd_qk(lib, Nq=2 ** 24 - 64, Nk=1, d=128) == -2           # the same for Q
    assert fwd_qk(lib, Nq=300, Nk=77, d=80) == -3
    assert fwd_qk(lib, o=P[1]) == -9                               # output aliases K
    assert bwd_qk(lib, Nq=0) == -2
    assert bwd_qk(lib, Nk=0) == -2
    assert bwd_qk(lib, Nq=33, Nk=1000, scale=float("nan")) == -7
    # the workspace is sized by the query length: one sized for N_k < N_q is refused
    big = lib.fa_bwd_workspace_size(1, 1, 512, 64)
    assert bwd_qk(lib, Nq=512, Nk=64, ws_bytes=lib.fa_bwd_workspace_size(1, 1, 64, 64)) == -6
    assert bwd_qk(lib, Nq=512, Nk=64, ws_bytes=big, scale=float("nan")) == -7


def fwd_ex(lib, H=4, Hkv=2, Nq=128, Nk=128, window=0, B=1, d=64, scale=0.125, causal=1, **ptrs):
    p = dict(q=P[0], k=P[1], v=P[2], o=P[3], lse=P[4])
    p.update(ptrs)
    return lib.fa_fwd_ex(p["q"], p["k"], p["v"], p["o"], p["lse"], B, H, Hkv, Nq, Nk, d, scale, causal,
                         window, None)


def bwd_ex(lib, H=4, Hkv=2, Nq=128, Nk=128, window=0, B=1, d=64, scale=0.125, causal=1, ws=P[9],
           ws_bytes=None, **ptrs):
    p = dict(q=P[0], k=P[1], v=P[2], o=P[3], lse=P[4], do=P[5], dq=P[6], dk=P[7], dv=P[8])
    p.update(ptrs)
    if ws_bytes is None:
        ws_bytes = lib.fa_bwd_workspace_size(B, H, Nq, d)
    return lib.fa_bwd_ex(p["q"], p["k"], p["v"], p["o"], p["lse"], p["do"], p["dq"], p["dk"], p["dv"],
                         B, H, Hkv, Nq, Nk, d, scale, causal, window, ws, ws_bytes, None)


def test_grouped_heads_and_window_validation(lib):
    nan = float("nan")
    for call in (fwd_ex, bwd_ex):
        assert call(lib, Hkv=0) == -2
        assert call(lib, Hkv=-1) == -2
        assert call(lib, H=6, Hkv=4) == -2                  # 6 query heads over 4 K/V heads
        assert call(lib, H=4, Hkv=8) == -2
        assert call(lib, window=-1) == -9
        assert call(lib, causal=0, window=-3) == -9
        assert call(lib, H=8, Hkv=1, scale=nan) == -7       # multi-query: valid shape
        assert call(lib, H=8, Hkv=8, window=1, scale=nan) == -7
        assert call(lib, H=32, Hkv=4, Nq=77, Nk=300, window=4096, causal=0, scale=nan) == -7
    # K / V are sized by H_kv: a K with more than 2^31 elements is refused even
    # when Q is small, and one under it is accepted
    assert fwd_ex(lib, H=16, Hkv=16, Nq=1, Nk=2 ** 20, d=128) == -2
    assert fwd_ex(lib, H=16, Hkv=1, Nq=1, Nk=2 ** 20, d=128, scale=nan) == -7
    # overlap checks use the K / V extent: B N_k H_kv d bf16 = 16 KiB here
    assert fwd_ex(lib, H=4, Hkv=1, o=P[1] + 16384 - 256) == -9
    assert fwd_ex(lib, H=4, Hkv=1, o=P[1] + 16384, scale=nan) == -7
    assert bwd_ex(lib, H=4, Hkv=1, dk=P[2] + 16384 - 256) == -9


def dec(lib, H=8, Hkv=2, Nq=1, Nk=4096, d=128, B=1, scale=0.125, causal=1, window=0, splits=0, ws=P[9],
        ws_bytes=None, **ptrs):
    p = dict(q=P[0], k=P[1], v=P[2], o=P[3], lse=P[4])
    p.update(ptrs)
    if ws_bytes is None:
        ws_bytes = lib.fa_decode_workspace_size(B, H, Hkv, Nq, Nk, d, causal, window, splits)
    return lib.fa_fwd_decode(p["q"], p["k"], p["v"], p["o"], p["lse"], B, H, Hkv, Nq, Nk, d, scale, causal,
                             window, splits, ws, ws_bytes, None)


def test_decode_workspace_size(lib):
    r256 = lambda x: (x + 255) // 256 * 256
    size = lib.fa_decode_workspace_size
    # 8 query heads over 2 key heads, one position, 4096 keys = 32 stages of
    # 128: 2 units of (batch, key head) would take 128 splits to fill 256
    # CUs, capped at 32 / 4 = 8 so each split keeps 4 stages
    assert size(1, 8, 2, 1, 4096, 128, 1, 0, 0) == r256(8 * 8 * 1 * 129 * 4)
    assert size(1, 8, 2, 1, 65536, 128, 1, 0, 0) == r256(128 * 8 * 129 * 4)   # 512 stages: 128 splits
    assert size(1, 8, 2, 1, 65536, 64, 1, 0, 0) == r256(128 * 8 * 65 * 4)     # d = 64: 256 -> capped 128
    assert size(4, 8, 8, 1, 65536, 128, 1, 0, 0) == r256(8 * 32 * 129 * 4)    # 32 units: 8 splits
    assert size(1, 8, 2, 1, 4096, 128, 1, 0, 5) == r256(5 * 8 * 129 * 4)      # as asked
    assert size(1, 8, 2, 1, 4096, 128, 1, 0, 99) == r256(32 * 8 * 129 * 4)    # at most one per stage
    assert size(1, 8, 2, 1, 4096, 128, 1, 0, 1) == 0              # one split: no partials
    assert size(1, 8, 2, 1, 100, 64, 1, 0, 0) == 0                # one stage of keys
    assert size(300, 8, 1, 1, 4096, 128, 1, 0, 0) == 0            # 300 units fill the GPU
    # a window of 256 keys at the end of 65536: keys 65280 .. 65535, 2 stages
    assert size(1, 8, 2, 1, 65536, 128, 1, 256, 2) == r256(2 * 8 * 129 * 4)
    assert size(1, 8, 2, 1, 65536, 128, 1, 256, 3) == r256(2 * 8 * 129 * 4)
    assert size(1, 8, 2, 1, 65536, 128, 1, 257, 3) == r256(3 * 8 * 129 * 4)  # one key more: 3 stages
    assert size(1, 64, 1, 1, 4096, 128, 1, 0, 0) == 0             # 64 rows per key head: not packed
    assert size(1, 8, 2, 1, 4096, 128, 1, 0, -1) == 0             # invalid
    assert size(1, 6, 4, 1, 4096, 128, 1, 0, 0) == 0              # invalid


def test_decode_validation(lib):
    nan = float("nan")
    assert dec(lib, q=None) == -1
    assert dec(lib, Hkv=3) == -2
    assert dec(lib, d=96) == -3
    assert dec(lib, o=P[3] + 8) == -5
    assert dec(lib, scale=nan) == -7
    assert dec(lib, splits=-1) == -9
    assert dec(lib, window=-1) == -9
    assert dec(lib, ws=None) == -6                                   # 32 splits need a workspace
    assert dec(lib, ws_bytes=100) == -6
    assert dec(lib, ws=P[9] + 64) == -6
    assert dec(lib, o=P[1]) == -9                                    # output aliases K
    assert dec(lib, ws=P[2]) == -9                                   # workspace aliases V
    assert dec(lib, splits=1, ws=None, ws_bytes=0, scale=nan) == -7   # one split needs no workspace


def test_workspace_size(lib):
    assert lib.fa_bwd_workspace_size(0, 1, 64, 64) == 0
    assert lib.fa_bwd_workspace_size(1, 1, 64, 80) == 0
    B, H, N, d = 4, 16, 4096, 128
    rows = B * H * N * 4 * 2          # D and -lse * log2(e), float32 each
    r256 = lambda x: (x + 255) // 256 * 256
    assert lib.fa_bwd_workspace_size(B, H, N, d) == r256(rows)
    assert lib.fa_bwd_workspace_size(1, 3, 64, 64) == r256(3 * 64 * 4 * 2)


def test_binding_input_checks():
    """The binding's checks of the tensors the C ABI cannot see; every
    other check passes first, so the last error is the device."""
    import torch

    from io_aware_tiled_fa_amd import binding

    q = torch.zeros(2, 64, 4, 64, dtype=torch.bfloat16)
    kv = torch.zeros(2, 80, 2, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="on the GPU"):
        binding.check_inputs(q, kv, kv)              # valid shapes, but on the CPU
    with pytest.raises(TypeError, match="dtype"):
        binding.check_inputs(q.float(), kv, kv)
    with pytest.raises(ValueError, match="dims"):
        binding.check_inputs(q[0], kv, kv)
    with pytest.raises(TypeError, match="not a torch.Tensor"):
        binding.check_inputs(q, kv.float().numpy(), kv)
    with pytest.raises(ValueError, match="share batch"):
        binding.check_inputs(q, kv[:1], kv[:1])      # batch differs
    with pytest.raises(ValueError, match="share batch"):
        binding.check_inputs(q, kv[..., :32], kv[..., :32])   # head_dim differs
    with pytest.raises(ValueError, match="share batch"):
        binding.check_inputs(q, torch.zeros(2, 80, 3, 64, dtype=torch.bfloat16), kv)  # 4 heads over 3
    with pytest.raises(ValueError, match="shape"):
        binding.check_inputs(q, kv, kv[:, :79])      # K and V lengths differ
    with pytest.raises(ValueError, match="contiguous"):
        binding.check_inputs(q, kv, kv.transpose(1, 2).contiguous().transpose(1, 2))


def test_binding_output_checks():
    """Caller-supplied outputs and workspaces are checked against the call's
    sizes, dtype, device and contiguity before any pointer reaches the C ABI."""
    import torch

    from io_aware_tiled_fa_amd import binding

    q = torch.zeros(2, 64, 4, 64, dtype=torch.bfloat16)
    kv = torch.zeros(2, 80, 2, 64, dtype=torch.bfloat16)
    shp = binding.AttentionShape(q, kv)
    cpu = q.device
    o, lse = binding._outputs(shp, cpu)
    assert tuple(o.shape) == (2, 64, 4, 64) and o.dtype == torch.bfloat16
    assert tuple(lse.shape) == (2, 4, 64) and lse.dtype == torch.float32
    with pytest.raises(ValueError, match="shape"):
        binding._outputs(shp, cpu, o=torch.zeros(2, 64, 4, 32, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="shape"):
        binding._outputs(shp, cpu, lse=torch.zeros(2, 4, 63))
    with pytest.raises(TypeError, match="dtype"):
        binding._outputs(shp, cpu, o=torch.zeros(2, 64, 4, 64))
    with pytest.raises(TypeError, match="dtype"):
        binding._outputs(shp, cpu, lse=torch.zeros(2, 4, 64, dtype=torch.float64))
    with pytest.raises(ValueError, match="contiguous"):
        binding._outputs(shp, cpu, lse=torch.zeros(2, 64, 4).transpose(1, 2))
    with pytest.raises(ValueError, match="is on"):
        binding._outputs(shp, torch.device("meta"), o=o)
    with pytest.raises(ValueError, match="needs 512"):
        binding._workspace(torch.zeros(100, dtype=torch.uint8), 512, cpu)
    with pytest.raises(TypeError, match="uint8"):
        binding._workspace(torch.zeros(512), 512, cpu)
    assert binding._workspace(None, 0, cpu) is None
    assert binding._workspace(None, 300, cpu).numel() == 300


def test_noalloc_validation(lib):
    """fa_bwd_noalloc validates like fa_bwd_ex and refuses problems beyond its
    static scratch (2^21 query rows) before any HIP call."""
    Q = [0x100000000 * (i + 1) for i in range(10)]  # 4 GiB apart: nothing overlaps
    args = dict(B=2048, H=1, Hkv=1, Nq=1024, Nk=64, d=64, scale=0.125, causal=1, window=0)

    def call(**kw):
        a = dict(args, **kw)
        return lib.fa_bwd_noalloc(*Q[:9], a["B"], a["H"], a["Hkv"], a["Nq"], a["Nk"], a["d"], a["scale"],
                                  a["causal"], a["window"], None)
    assert call(B=2049) == -10                       # 2^21 + 1024 rows
    assert call(scale=float("nan")) == -7            # 2^21 rows fit
    assert call(d=96) == -3
    assert call(Hkv=3, H=4) == -2
    assert call(window=-1) == -9
    assert lib.fa_bwd_noalloc(None, *Q[1:9], 1, 1, 1, 64, 64, 64, 0.125, 1, 0, None) == -1
