"""Size of the score matrix that standard attention would materialise.

TEST INFRASTRUCTURE ONLY (see the package docstring).

"What Is Flash Attention? The Real Speed and Memory Gains, Explained"
(bestllmfor.com), section "The problem: a matrix that grows with the square
of the context", computes the transient score matrix of naive attention as
N x N entries per head at 2 bytes each (FP16), times the number of heads for
a layer.  FlashAttention never allocates it; the kernels' HBM traffic is
linear in N instead.
"""

from __future__ import annotations


def naive_score_bytes(n: int, heads: int = 1, bytes_per_element: int = 2) -> int:
    """Bytes of an N x N score matrix for ``heads`` heads."""
    return int(n) * int(n) * int(bytes_per_element) * int(heads)
