"""Seeded synthetic inputs shared by the HIP path, the oracle and the tests.

This module draws random numbers and rounds them to bfloat16. It holds none
of the attention arithmetic, so both sides of a parity check can take their
inputs from it without sharing any of the method.

Recipe (the pages' workload is long-prompt prefill on [batch, seq_len,
num_heads, head_dim] tensors, holysheep.ai review, "Implementing Flash
Attention in Your Architecture" code block; no dataset is named, so i.i.d.
normal tensors stand in for real activations):

* generator: ``numpy.random.default_rng(seed)`` (PCG64), seed 0 by default;
* tensors drawn in the order Q, K, V, then dO when a backward input is asked
  for, each as ``standard_normal((B, N, H, d), dtype=float32)`` (K and V use
  ``N_k`` rows when it differs from ``N``, and ``H_kv`` heads when it
  differs from ``H``);
* optional "peaked rows": after all tensors are drawn, for every (b, h) in
  row-major order, ``round(fraction * N)`` distinct query positions are chosen
  with ``rng.choice(N, size, replace=False)`` and those Q rows are multiplied
  by ``peak_factor`` (4 by default, exact in bfloat16);
* every tensor is rounded float32 -> bfloat16 with round-to-nearest-even.

The bfloat16 values are returned two ways: as raw ``uint16`` bit patterns
(what device memory holds) and as float32 arrays holding exactly the same
values (every bfloat16 is a float32), which the oracle upcasts to float64.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round to nearest, ties to even); return bits.

    bfloat16 is the upper 16 bits of an IEEE binary32.  Rounding adds
    0x7FFF plus the lowest kept bit to the 32-bit pattern before truncation,
    which is the integer form of round-half-to-even.  NaNs are kept quiet
    NaNs instead of being carried into the exponent.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    rounded = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    nan = np.isnan(x)
    if nan.any():
        rounded = np.where(nan, (u >> np.uint32(16)) | np.uint32(0x0040), rounded)
    return rounded.astype(np.uint16)


def f32_from_bf16_bits(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclass
class AttentionInputs:
    """One seeded problem instance, BSHD layout throughout."""

    B: int
    H: int
    N: int
    d: int
    N_k: int
    seed: int
    H_kv: int
    q_bits: np.ndarray
    k_bits: np.ndarray
    v_bits: np.ndarray
    do_bits: Optional[np.ndarray] = None
    peaked_rows: Optional[np.ndarray] = None  # [B, H, n_peaked] query indices
    _cache: dict = field(default_factory=dict, repr=False)

    def values(self, name: str) -> np.ndarray:
        """float32 array with exactly the bfloat16 values of tensor ``name``."""
        if name not in self._cache:
            bits = getattr(self, name + "_bits")
            if bits is None:
                raise KeyError(name)
            self._cache[name] = f32_from_bf16_bits(bits)
        return self._cache[name]

    @property
    def q(self) -> np.ndarray:
        return self.values("q")

    @property
    def k(self) -> np.ndarray:
        return self.values("k")

    @property
    def v(self) -> np.ndarray:
        return self.values("v")

    @property
    def do(self) -> np.ndarray:
        return self.values("do")


def make_inputs(B: int, H: int, N: int, d: int, *, seed: int = 0,
                N_k: Optional[int] = None, H_kv: Optional[int] = None, with_do: bool = False,
                peaked_fraction: float = 0.0,
                peak_factor: float = 4.0) -> AttentionInputs:
    """Draw Q, K, V (and dO) as described in the module docstring."""
    if N_k is None:
        N_k = N
    if H_kv is None:
        H_kv = H
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, N, H, d), dtype=np.float32)
    k = rng.standard_normal((B, N_k, H_kv, d), dtype=np.float32)
    v = rng.standard_normal((B, N_k, H_kv, d), dtype=np.float32)
    do = rng.standard_normal((B, N, H, d), dtype=np.float32) if with_do else None
    peaked = None
    if peaked_fraction > 0.0:
        count = int(round(peaked_fraction * N))
        peaked = np.empty((B, H, count), dtype=np.int64)
        for b in range(B):
            for h in range(H):
                rows = rng.choice(N, size=count, replace=False)
                peaked[b, h] = rows
                q[b, rows, h, :] *= np.float32(peak_factor)
    return AttentionInputs(
        B=B, H=H, N=N, d=d, N_k=N_k, seed=seed, H_kv=H_kv,
        q_bits=bf16_bits_from_f32(q), k_bits=bf16_bits_from_f32(k),
        v_bits=bf16_bits_from_f32(v),
        do_bits=None if do is None else bf16_bits_from_f32(do),
        peaked_rows=peaked)


# The five workloads the kernels are held to.  Scale is 1/sqrt(d) in each
# (the pages' default when no softmax scale is given, holysheep.ai review,
# "Implementing Flash Attention in Your Architecture" code block).
WORKLOADS = {
    "fwd_b1_h1_n128_d64": dict(B=1, H=1, N=128, d=64, causal=False, kind="fwd"),
    "fwd_b4_h16_n2048_d64": dict(B=4, H=16, N=2048, d=64, causal=False, kind="fwd"),
    "fwd_b2_h32_n8192_d128_causal_peaked": dict(B=2, H=32, N=8192, d=128, causal=True,
                                                kind="fwd", peaked_fraction=0.01),
    "fwd_b1_h32_n32768_d128_causal": dict(B=1, H=32, N=32768, d=128, causal=True, kind="fwd"),
    "bwd_b4_h16_n4096_d128_causal": dict(B=4, H=16, N=4096, d=128, causal=True, kind="bwd"),
}


def make_workload(name: str, seed: int = 0) -> AttentionInputs:
    w = WORKLOADS[name]
    return make_inputs(w["B"], w["H"], w["N"], w["d"], seed=seed,
                       with_do=(w["kind"] == "bwd"),
                       peaked_fraction=w.get("peaked_fraction", 0.0))
