"""Thin ctypes binding of libfa.so (include/fa.h).

Argument marshalling only: torch supplies device memory and the current HIP
stream; every step of attention runs in the library's kernels.  There is no
fallback: if libfa.so is missing or a call fails, an exception is raised.

Each call goes to the narrowest entry point that covers it: fa_fwd / fa_bwd
for self-attention (N_q = N_k, one K/V head per query head, no window),
fa_fwd_qk / fa_bwd_qk when only the lengths differ, fa_fwd_ex / fa_bwd_ex
otherwise.

The checks here restate the layout the C ABI documents (Q, O, dO, dQ as
[B, N_q, H, d]; K, V, dK, dV as [B, N_k, H_kv, d]; LSE as [B, H, N_q]) in
terms of torch tensors, plus what the library cannot check from raw
pointers: dtypes, contiguity, the device, and the extent of every tensor
the caller hands in, outputs included (a wrong-sized output would let a
kernel write past it).  The pages' interface takes [batch, seq_len,
num_heads, head_dim] tensors with a common batch, head dimension and K/V
length (holysheep.ai review, "Common Errors and Fixes", Error 4).
"""

from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Tuple

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libfa.so")

FA_STATUS = {
    0: "FA_OK", -1: "FA_ERR_NULL", -2: "FA_ERR_SHAPE", -3: "FA_ERR_HEADDIM",
    -4: "FA_ERR_SEQLEN", -5: "FA_ERR_ALIGN", -6: "FA_ERR_WORKSPACE",
    -7: "FA_ERR_SCALE", -8: "FA_ERR_LAUNCH", -9: "FA_ERR_ARG", -10: "FA_ERR_SCRATCH",
}
EXPORTED = ("fa_fwd", "fa_fwd_qk", "fa_fwd_ex", "fa_fwd_decode", "fa_decode_workspace_size", "fa_bwd",
            "fa_bwd_qk", "fa_bwd_ex", "fa_bwd_noalloc", "fa_bwd_workspace_size", "fa_status_string", "fa_version")

_lib = None


class FAError(RuntimeError):
    def __init__(self, fn: str, status: int, text: str):
        super().__init__(f"{fn} failed: {FA_STATUS.get(status, status)} ({text})")
        self.status = status


def load_library(path: Optional[str] = None) -> ctypes.CDLL:
    """Load libfa.so and declare its signatures (raises if it is not built)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is missing; build it with `python -m io_aware_tiled_fa_amd.build`")
    lib = ctypes.CDLL(p)
    vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.fa_fwd.restype = i
    lib.fa_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, vp]
    lib.fa_bwd.restype = i
    lib.fa_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, f, i, vp, sz, vp]
    lib.fa_fwd_qk.restype = i
    lib.fa_fwd_qk.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp]
    lib.fa_bwd_qk.restype = i
    lib.fa_bwd_qk.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp, sz, vp]
    lib.fa_fwd_ex.restype = i
    lib.fa_fwd_ex.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, i, vp]
    lib.fa_bwd_ex.restype = i
    lib.fa_bwd_ex.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, i, vp, sz, vp]
    lib.fa_bwd_noalloc.restype = i
    lib.fa_bwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, i, vp]
    lib.fa_fwd_decode.restype = i
    lib.fa_fwd_decode.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, i, i, vp, sz, vp]
    lib.fa_decode_workspace_size.restype = sz
    lib.fa_decode_workspace_size.argtypes = [i, i, i, i, i, i, i, i, i]
    lib.fa_bwd_workspace_size.restype = sz
    lib.fa_bwd_workspace_size.argtypes = [i, i, i, i]
    lib.fa_status_string.restype = ctypes.c_char_p
    lib.fa_status_string.argtypes = [i]
    lib.fa_version.restype = i
    lib.fa_version.argtypes = []
    if path is None:
        _lib = lib
    return lib


def _check(lib, fn: str, status: int):
    if status != 0:
        raise FAError(fn, status, lib.fa_status_string(status).decode())


class AttentionShape:
    """B, N_q, N_k, H, H_kv, d of one call, read off Q and K."""

    def __init__(self, q, k):
        self.B, self.Nq, self.H, self.d = (int(x) for x in q.shape)
        self.Nk, self.Hkv = int(k.shape[1]), int(k.shape[2])

    @property
    def q_like(self):
        return (self.B, self.Nq, self.H, self.d)

    @property
    def kv_like(self):
        return (self.B, self.Nk, self.Hkv, self.d)

    @property
    def rows(self):
        return (self.B, self.H, self.Nq)


def _expect(t, what: str, shape, dtype, device) -> None:
    """Raise unless ``t`` is a contiguous ``dtype`` tensor of ``shape`` on
    ``device`` (``what`` names the argument in the error)."""
    import torch

    if not isinstance(t, torch.Tensor):
        raise TypeError(f"fa: {what} is a {type(t).__name__}, not a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"fa: {what} has dtype {t.dtype}; the library takes {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"fa: {what} has shape {tuple(t.shape)}; this call needs {tuple(shape)}")
    if t.device != device:
        raise ValueError(f"fa: {what} is on {t.device}, the other tensors on {device}")
    if not t.is_contiguous():
        raise ValueError(f"fa: {what} is not contiguous; the library reads plain row-major memory")


def check_inputs(q, k, v) -> AttentionShape:
    """Check Q [B, N_q, H, d] and K, V [B, N_k, H_kv, d] (bf16, contiguous,
    one GPU; H a multiple of H_kv) and return the call's sizes."""
    import torch

    for what, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"fa: {what} is a {type(t).__name__}, not a torch.Tensor")
        if t.dim() != 4:
            raise ValueError(f"fa: {what} has {t.dim()} dims; tensors are [batch, seq_len, heads, head_dim]")
    if q.shape[0] != k.shape[0] or q.shape[3] != k.shape[3] or k.shape[2] == 0 or q.shape[2] % k.shape[2]:
        raise ValueError(f"fa: q {tuple(q.shape)} and k {tuple(k.shape)} must share batch and head_dim, "
                         "and k's heads must divide q's")
    shp = AttentionShape(q, k)
    _expect(q, "q", shp.q_like, torch.bfloat16, q.device)
    _expect(k, "k", shp.kv_like, torch.bfloat16, q.device)
    _expect(v, "v", shp.kv_like, torch.bfloat16, q.device)
    if not q.is_cuda:
        raise ValueError(f"fa: the tensors are on {q.device}; the library runs on the GPU")
    return shp


def _stream_ptr(device, stream) -> int:
    import torch

    if stream is None:
        stream = torch.cuda.current_stream(device)
    return int(stream.cuda_stream)


def default_scale(head_dim: int) -> float:
    """1 / sqrt(head_dim), the default softmax scale of the pages' interface."""
    return 1.0 / math.sqrt(head_dim)


def _outputs(shp: AttentionShape, device, o=None, lse=None):
    """The caller's O and LSE after checking them, or fresh ones."""
    import torch

    if o is None:
        o = torch.empty(shp.q_like, dtype=torch.bfloat16, device=device)
    else:
        _expect(o, "out", shp.q_like, torch.bfloat16, device)
    if lse is None:
        lse = torch.empty(shp.rows, dtype=torch.float32, device=device)
    else:
        _expect(lse, "lse", shp.rows, torch.float32, device)
    return o, lse


def forward(q, k, v, causal: bool = False, scale: Optional[float] = None, window: int = 0,
            out=None, lse=None, stream=None) -> Tuple[object, object]:
    """O, LSE of attention: Q bf16 [B, N_q, H, d], K and V bf16
    [B, N_k, H_kv, d] on the GPU (N_q = N_k and H_kv = H is plain
    self-attention; H_kv < H is grouped-query attention).  window > 0 limits
    each query to the keys within that distance of its position."""
    shp = check_inputs(q, k, v)
    if scale is None:
        scale = default_scale(shp.d)
    out, lse = _outputs(shp, q.device, out, lse)
    lib = load_library()
    ptrs = (q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr())
    flags = (float(scale), int(bool(causal)))
    strm = _stream_ptr(q.device, stream)
    if shp.Hkv == shp.H and window == 0 and shp.Nq == shp.Nk:
        fn, st = "fa_fwd", lib.fa_fwd(*ptrs, shp.B, shp.H, shp.Nq, shp.d, *flags, strm)
    elif shp.Hkv == shp.H and window == 0:
        fn, st = "fa_fwd_qk", lib.fa_fwd_qk(*ptrs, shp.B, shp.H, shp.Nq, shp.Nk, shp.d, *flags, strm)
    else:
        fn, st = "fa_fwd_ex", lib.fa_fwd_ex(*ptrs, shp.B, shp.H, shp.Hkv, shp.Nq, shp.Nk, shp.d, *flags,
                                            int(window), strm)
    _check(lib, fn, st)
    return out, lse


def decode(q, k, v, causal: bool = False, scale: Optional[float] = None, window: int = 0,
           num_splits: int = 0, out=None, lse=None, workspace=None, stream=None) -> Tuple[object, object]:
    """O, LSE = fa_fwd_decode(Q, K, V): the split-KV forward for few query
    rows against a long key sequence (same arguments and results as
    forward, plus the number of key splits, 0 = the library's choice)."""
    import torch

    shp = check_inputs(q, k, v)
    if scale is None:
        scale = default_scale(shp.d)
    out, lse = _outputs(shp, q.device, out, lse)
    lib = load_library()
    need = int(lib.fa_decode_workspace_size(shp.B, shp.H, shp.Hkv, shp.Nq, shp.Nk, shp.d, int(bool(causal)),
                                            int(window), int(num_splits)))
    workspace = _workspace(workspace, need, q.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() if workspace is not None else 0
    st = lib.fa_fwd_decode(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                           shp.B, shp.H, shp.Hkv, shp.Nq, shp.Nk, shp.d, float(scale), int(bool(causal)),
                           int(window), int(num_splits), ws_ptr, ws_bytes, _stream_ptr(q.device, stream))
    _check(lib, "fa_fwd_decode", st)
    return out, lse


def _workspace(ws, need: int, device):
    """The caller's workspace (a uint8 device tensor of at least ``need``
    bytes) or a fresh one; None when nothing is needed and none was given."""
    import torch

    if ws is None:
        return torch.empty(need, dtype=torch.uint8, device=device) if need > 0 else None
    if not isinstance(ws, torch.Tensor) or ws.dtype != torch.uint8 or ws.dim() != 1:
        raise TypeError("fa: workspace must be a one-dimensional uint8 tensor")
    if ws.device != device or not ws.is_contiguous():
        raise ValueError(f"fa: workspace must be contiguous and on {device}")
    if ws.numel() < need:
        raise ValueError(f"fa: workspace holds {ws.numel()} bytes; this call needs {need}")
    return ws


def bwd_workspace_size(B: int, H: int, N: int, d: int) -> int:
    return int(load_library().fa_bwd_workspace_size(B, H, N, d))


def backward(q, k, v, o, lse, do, causal: bool = False, scale: Optional[float] = None, window: int = 0,
             dq=None, dk=None, dv=None, workspace=None, stream=None):
    """dQ, dK, dV of attention; O and LSE are the forward's outputs for the
    same arguments, dO the gradient of the loss with respect to O."""
    import torch

    shp = check_inputs(q, k, v)
    dev = q.device
    _expect(o, "o", shp.q_like, torch.bfloat16, dev)
    _expect(do, "do", shp.q_like, torch.bfloat16, dev)
    _expect(lse, "lse", shp.rows, torch.float32, dev)
    grads = []
    for what, t, like in (("dq", dq, shp.q_like), ("dk", dk, shp.kv_like), ("dv", dv, shp.kv_like)):
        if t is None:
            t = torch.empty(like, dtype=torch.bfloat16, device=dev)
        else:
            _expect(t, what, like, torch.bfloat16, dev)
        grads.append(t)
    dq, dk, dv = grads
    if scale is None:
        scale = default_scale(shp.d)
    lib = load_library()
    workspace = _workspace(workspace, int(lib.fa_bwd_workspace_size(shp.B, shp.H, shp.Nq, shp.d)), dev)
    ptrs = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), do.data_ptr(),
            dq.data_ptr(), dk.data_ptr(), dv.data_ptr())
    flags = (float(scale), int(bool(causal)))
    tail = (workspace.data_ptr(), workspace.numel(), _stream_ptr(dev, stream))
    if shp.Hkv == shp.H and window == 0 and shp.Nq == shp.Nk:
        fn, st = "fa_bwd", lib.fa_bwd(*ptrs, shp.B, shp.H, shp.Nq, shp.d, *flags, *tail)
    elif shp.Hkv == shp.H and window == 0:
        fn, st = "fa_bwd_qk", lib.fa_bwd_qk(*ptrs, shp.B, shp.H, shp.Nq, shp.Nk, shp.d, *flags, *tail)
    else:
        fn, st = "fa_bwd_ex", lib.fa_bwd_ex(*ptrs, shp.B, shp.H, shp.Hkv, shp.Nq, shp.Nk, shp.d, *flags,
                                            int(window), *tail)
    _check(lib, fn, st)
    return dq, dk, dv
