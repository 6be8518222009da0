"""The fp64 oracle against its pins (closed forms, invariants, finite
differences, brute force, torch float64).  CPU only."""

import pytest

import oracle
from oracle_pins import ALL_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=[p.__name__ for p in ALL_PINS])
def test_oracle_pin(pin):
    pin(oracle)
