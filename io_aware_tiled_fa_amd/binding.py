"""Thin ctypes binding of libfa.so (include/fa.h).

Argument marshalling only: torch supplies device memory and the current HIP
stream; every step of attention runs in the library's kernels.  There is no
fallback: if libfa.so is missing or a call fails, an exception is raised.

The checks in :func:`validate_attention_inputs` follow the interface checks
of the holysheep.ai review ("Common Errors and Fixes", Error 4: 4-D
[batch, seq_len, num_heads, head_dim] tensors, equal batch, heads and
head_dim, equal K and V lengths), plus what the kernels need (bfloat16,
contiguous, on the GPU, one sequence length).
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
    -7: "FA_ERR_SCALE", -8: "FA_ERR_LAUNCH", -9: "FA_ERR_ARG",
}
EXPORTED = ("fa_fwd", "fa_fwd_qk", "fa_fwd_ex", "fa_fwd_decode", "fa_decode_workspace_size", "fa_bwd",
            "fa_bwd_qk", "fa_bwd_ex", "fa_bwd_workspace_size", "fa_status_string", "fa_version")

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


def validate_attention_inputs(q, k, v) -> None:
    import torch

    for name, t in (("Q", q), ("K", k), ("V", v)):
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch.Tensor")
        if t.dim() != 4:
            raise ValueError(f"{name} must have 4 dimensions [batch, seq_len, num_heads, head_dim], got {t.dim()}")
        if t.dtype != torch.bfloat16:
            raise TypeError(f"{name} must be bfloat16, got {t.dtype}")
        if not t.is_cuda:
            raise ValueError(f"{name} must be on the GPU")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if not (q.shape[0] == k.shape[0] == v.shape[0]):
        raise ValueError(f"Batch size mismatch: Q={q.shape[0]}, K={k.shape[0]}, V={v.shape[0]}")
    if k.shape[2] != v.shape[2] or q.shape[2] % k.shape[2] != 0:
        raise ValueError(f"Num heads mismatch: Q={q.shape[2]}, K={k.shape[2]}, V={v.shape[2]} "
                         "(K and V need equal heads, and Q a multiple of them)")
    if k.shape[1] != v.shape[1]:
        raise ValueError(f"Key/Value sequence length mismatch: K={k.shape[1]}, V={v.shape[1]}")
    if not (q.shape[3] == k.shape[3] == v.shape[3]):
        raise ValueError(f"Head dimension mismatch: Q={q.shape[3]}, K={k.shape[3]}, V={v.shape[3]}")
    if not (q.device == k.device == v.device):
        raise ValueError("Q, K and V must be on one device")


def _stream_ptr(device, stream) -> int:
    import torch

    if stream is None:
        stream = torch.cuda.current_stream(device)
    return int(stream.cuda_stream)


def default_scale(head_dim: int) -> float:
    """1 / sqrt(head_dim), the default softmax scale of the pages' interface."""
    return 1.0 / math.sqrt(head_dim)


def forward(q, k, v, causal: bool = False, scale: Optional[float] = None, window: int = 0,
            out=None, lse=None, stream=None) -> Tuple[object, object]:
    """O, LSE = fa_fwd_ex(Q, K, V); Q bf16 [B, N_q, H, d], K and V bf16
    [B, N_k, H_kv, d] on the GPU (N_q = N_k and H_kv = H is plain
    self-attention; H_kv < H is grouped-query attention).  window > 0 limits
    each query to the keys within that distance of its position."""
    import torch

    validate_attention_inputs(q, k, v)
    B, Nq, H, d = q.shape
    Nk, Hkv = k.shape[1], k.shape[2]
    if scale is None:
        scale = default_scale(d)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    lib = load_library()
    st = lib.fa_fwd_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                       B, H, Hkv, Nq, Nk, d, float(scale), int(bool(causal)), int(window),
                       _stream_ptr(q.device, stream))
    _check(lib, "fa_fwd_ex", st)
    return out, lse


def decode(q, k, v, causal: bool = False, scale: Optional[float] = None, window: int = 0,
           num_splits: int = 0, out=None, lse=None, workspace=None, stream=None) -> Tuple[object, object]:
    """O, LSE = fa_fwd_decode(Q, K, V): the split-KV forward for few query
    rows against a long key sequence (same arguments and results as
    forward, plus the number of key splits, 0 = the library's choice)."""
    import torch

    validate_attention_inputs(q, k, v)
    B, Nq, H, d = q.shape
    Nk, Hkv = k.shape[1], k.shape[2]
    if scale is None:
        scale = default_scale(d)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    lib = load_library()
    need = int(lib.fa_decode_workspace_size(B, H, Hkv, Nq, Nk, d, int(bool(causal)), int(window), int(num_splits)))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = lib.fa_fwd_decode(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                           B, H, Hkv, Nq, Nk, d, float(scale), int(bool(causal)), int(window), int(num_splits),
                           ws_ptr, ws_bytes, _stream_ptr(q.device, stream))
    _check(lib, "fa_fwd_decode", st)
    return out, lse


def bwd_workspace_size(B: int, H: int, N: int, d: int) -> int:
    return int(load_library().fa_bwd_workspace_size(B, H, N, d))


def backward(q, k, v, o, lse, do, causal: bool = False, scale: Optional[float] = None, window: int = 0,
             dq=None, dk=None, dv=None, workspace=None, stream=None):
    """dQ, dK, dV = fa_bwd_ex(...); O and LSE are the forward's outputs."""
    import torch

    validate_attention_inputs(q, k, v)
    for name, t in (("O", o), ("dO", do)):
        if t.shape != q.shape or t.dtype != torch.bfloat16 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous bf16 tensor shaped like Q")
    B, N, H, d = q.shape
    Nk, Hkv = k.shape[1], k.shape[2]
    if lse.shape != (B, H, N) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("LSE must be a contiguous float32 [B, H, N_q] tensor")
    if scale is None:
        scale = default_scale(d)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    lib = load_library()
    need = int(lib.fa_bwd_workspace_size(B, H, N, d))
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    st = lib.fa_bwd_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                       do.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                       B, H, Hkv, N, Nk, d, float(scale), int(bool(causal)), int(window),
                       workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                       _stream_ptr(q.device, stream))
    _check(lib, "fa_bwd_ex", st)
    return dq, dk, dv
