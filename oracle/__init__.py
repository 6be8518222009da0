"""fp64 CPU oracle for exact attention.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the HIP library or its binding.
"""

from .attention import (  # noqa: F401
    attention_backward,
    attention_forward,
    head_backward,
    head_forward,
    row_softmax,
    scaled_scores,
    visible_mask,
)
from .sizes import naive_score_bytes  # noqa: F401
