"""A seeded sweep of small random problems: forward and backward through the
C ABI (fa_fwd_ex / fa_bwd_ex), and split-KV decoding (fa_fwd_decode),
against the fp64 oracle.

The fixed cases of the other modules pick their shapes by hand; these are
drawn once from a fixed generator so that row and key counts land anywhere
in a tile (including 1), with grouped K/V heads, both head dimensions,
causal or not, and sliding windows of any width.  Every launch shape the
small grids reach is exercised: the 4- and 8-wave forward kernels, the dQ
and dK/dV kernels, ragged first and last tiles, rows that see no key, and
the epilogues' partial row blocks.  The decoding draws pack up to 32 query
rows per key head, reach any key length and split count, and end their
stages ragged.  Comparison rules: gpu_checks.py.
"""

import math

import numpy as np
import pytest

from gpu_checks import check_backward, check_decode
from io_aware_tiled_fa_amd.inputs import make_inputs
from parity import announce


def _draw_cases(count: int, seed: int):
    rng = np.random.default_rng(seed)
    cases = []
    for _ in range(count):
        Hkv = int(rng.choice([1, 2, 4]))
        G = int(rng.choice([1, 2, 4]))
        B = int(rng.integers(1, 3))
        d = int(rng.choice([64, 128]))
        # lengths: 1 .. 4, just off a tile edge, or uniform over 1 .. 600
        def length():
            u = rng.random()
            if u < 0.15:
                return int(rng.integers(1, 5))
            if u < 0.45:
                return int(rng.choice([32, 64, 128, 256, 384])) + int(rng.integers(-1, 2))
            return int(rng.integers(1, 601))
        Nq, Nk = length(), length()
        causal = bool(rng.random() < 0.6)
        window = int(rng.integers(1, Nk + 1)) if rng.random() < 0.3 else 0
        cases.append((B, Hkv * G, Hkv, Nq, Nk, d, causal, window))
    return cases


# the draw, plus the smallest problems by hand: one query row against many
# keys, a 1 x 1 problem, and causal rows of which all but the last see no key
CASES = _draw_cases(24, seed=20261203) + [
    (1, 4, 2, 1, 300, 128, True, 0),
    (1, 2, 2, 1, 1, 64, False, 0),
    (2, 4, 4, 5, 1, 128, True, 0),
]


def _draw_decode_cases(count: int, seed: int):
    rng = np.random.default_rng(seed)
    cases = []
    for _ in range(count):
        Hkv = int(rng.choice([1, 2, 4]))
        G = int(rng.choice([1, 2, 4, 8]))
        Nq = int(rng.integers(1, 32 // G + 1))  # the packed tile holds G N_q <= 32 rows
        B = int(rng.integers(1, 3))
        d = int(rng.choice([64, 128]))
        Nk = int(rng.integers(1, 20001)) if rng.random() < 0.7 else int(rng.integers(1, 300))
        causal = bool(rng.random() < 0.7)
        window = int(rng.integers(1, Nk + 1)) if rng.random() < 0.3 else 0
        splits = int(rng.choice([0, 0, 1, 2, 5, 64]))
        cases.append((B, Hkv * G, Hkv, Nq, Nk, d, causal, window, splits))
    return cases


# the draw, plus full 32-row tiles: eight query heads per key head at four
# positions, and 32 heads on one K/V head with more splits asked than stages
DECODE_CASES = _draw_decode_cases(16, seed=20261204) + [
    (2, 32, 4, 4, 3000, 64, True, 0, 0),
    (1, 32, 1, 1, 5000, 128, True, 0, 64),
]


@pytest.fixture(scope="module")
def fa():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from io_aware_tiled_fa_amd import binding

    binding.load_library()
    return binding


def test_cases_cover_the_edges():
    """The draw reaches every kind of case the docstring promises (no GPU)."""
    assert any(c[3] == 1 for c in CASES) and any(c[4] == 1 for c in CASES)
    assert {c[5] for c in CASES} == {64, 128}
    assert any(c[1] != c[2] for c in CASES)  # grouped K/V heads
    assert any(c[7] > 0 for c in CASES) and any(c[7] == 0 for c in CASES)
    assert any(c[6] for c in CASES) and any(not c[6] for c in CASES)
    assert any(c[3] > c[4] and c[6] for c in CASES)  # causal rows that see no key


@pytest.mark.gpu
@pytest.mark.parametrize("B,H,Hkv,Nq,Nk,d,causal,window", CASES)
def test_random_shape(fa, B, H, Hkv, Nq, Nk, d, causal, window):
    announce(f"random B={B} H={H} Hkv={Hkv} Nq={Nq} Nk={Nk} d={d} causal={causal} W={window}")
    inp = make_inputs(B, H, Nq, d, N_k=Nk, H_kv=Hkv, seed=9000 + Nq * 7 + Nk + window, with_do=True)
    check_backward(fa, inp, causal, 1.0 / math.sqrt(d), window)


def test_decode_cases_cover_the_edges():
    """The decoding draw reaches full 32-row tiles, forced splits and both head
    dimensions (no GPU)."""
    assert any(c[1] // c[2] * c[3] == 32 for c in DECODE_CASES)
    assert all(c[1] // c[2] * c[3] <= 32 for c in DECODE_CASES)
    assert {c[5] for c in DECODE_CASES} == {64, 128}
    assert any(c[8] == 1 for c in DECODE_CASES) and any(c[8] == 0 for c in DECODE_CASES)
    assert any(c[7] > 0 for c in DECODE_CASES)


@pytest.mark.gpu
@pytest.mark.parametrize("B,H,Hkv,Nq,Nk,d,causal,window,splits", DECODE_CASES)
def test_random_decode(fa, B, H, Hkv, Nq, Nk, d, causal, window, splits):
    announce(f"random decode B={B} H={H} Hkv={Hkv} Nq={Nq} Nk={Nk} d={d} causal={causal} W={window} "
             f"splits={splits}")
    inp = make_inputs(B, H, Nq, d, N_k=Nk, H_kv=Hkv, seed=9500 + Nq * 13 + Nk + window + splits)
    check_decode(fa, inp, causal, 1.0 / math.sqrt(d), window, splits)
