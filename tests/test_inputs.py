"""The seeded input generator: reproducibility and bfloat16 rounding."""

import numpy as np
import pytest

from io_aware_tiled_fa_amd.inputs import (WORKLOADS, bf16_bits_from_f32,
                                          f32_from_bf16_bits, make_inputs)


def _rne_reference(x):
    """bfloat16 RNE by exact rational rounding in float64 (independent form)."""
    out = np.empty(x.shape, dtype=np.uint16)
    for idx, val in np.ndenumerate(x.astype(np.float64)):
        if val == 0.0:
            out[idx] = 0x8000 if np.signbit(val) else 0
            continue
        m, e = np.frexp(abs(val))        # val = m * 2^e, m in [0.5, 1)
        # bf16 keeps 8 significant bits: round m * 2^8 to an integer, ties even
        scaled = m * 256.0
        r = np.floor(scaled)
        frac = scaled - r
        if frac > 0.5 or (frac == 0.5 and int(r) % 2 == 1):
            r += 1
        y = np.float32(np.ldexp(r / 256.0, e) * (-1 if val < 0 else 1))
        out[idx] = np.frombuffer(y.tobytes(), dtype=np.uint32)[0] >> 16
    return out


def test_bf16_rne_matches_rational_rounding():
    rng = np.random.default_rng(5)
    x = rng.standard_normal(4000).astype(np.float32) * np.float32(3.0)
    # include exact ties: values halfway between two bf16 numbers
    # (normal range: the rational form below assumes 8 significant bits)
    ties = ((np.arange(0x3E00, 0x3E00 + 200, dtype=np.uint32) << 16)
            | np.uint32(0x8000)).view(np.float32)
    x = np.concatenate([x, ties, -ties, np.float32([0.0, 1.0, -2.5, 65504.0])])
    assert np.array_equal(bf16_bits_from_f32(x), _rne_reference(x))


def test_bf16_roundtrip_exact():
    bits = np.arange(0, 0x7F80, 7, dtype=np.uint16)
    assert np.array_equal(bf16_bits_from_f32(f32_from_bf16_bits(bits)), bits)


def test_bf16_nan_stays_nan():
    x = np.array([np.nan, -np.nan], dtype=np.float32)
    assert np.isnan(f32_from_bf16_bits(bf16_bits_from_f32(x))).all()


def test_inputs_are_reproducible_and_ordered():
    a = make_inputs(2, 3, 40, 16, seed=0, with_do=True)
    b = make_inputs(2, 3, 40, 16, seed=0, with_do=True)
    for name in ("q", "k", "v", "do"):
        assert np.array_equal(getattr(a, name + "_bits"), getattr(b, name + "_bits"))
    rng = np.random.default_rng(0)
    q = rng.standard_normal((2, 40, 3, 16), dtype=np.float32)
    assert np.array_equal(a.q_bits, bf16_bits_from_f32(q))
    # Q, K, V drawn in that order from one stream; dO does not change them
    c = make_inputs(2, 3, 40, 16, seed=0, with_do=False)
    assert np.array_equal(a.v_bits, c.v_bits)


def test_peaked_rows():
    base = make_inputs(2, 2, 300, 8, seed=0)
    pk = make_inputs(2, 2, 300, 8, seed=0, peaked_fraction=0.01)
    assert pk.peaked_rows.shape == (2, 2, 3)
    for b in range(2):
        for h in range(2):
            rows = pk.peaked_rows[b, h]
            assert len(set(rows.tolist())) == 3
            mask = np.zeros(300, bool)
            mask[rows] = True
            np.testing.assert_array_equal(pk.q[b, mask, h], 4.0 * base.q[b, mask, h])
            np.testing.assert_array_equal(pk.q[b, ~mask, h], base.q[b, ~mask, h])
    np.testing.assert_array_equal(pk.k, base.k)


def test_workload_table():
    assert WORKLOADS["fwd_b2_h32_n8192_d128_causal_peaked"]["peaked_fraction"] == 0.01
    assert round(0.01 * 8192) == 82
    names = list(WORKLOADS)
    assert len(names) == 5
