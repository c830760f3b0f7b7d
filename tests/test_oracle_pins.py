"""The oracle against its pins (CPU only)."""

import pytest

import oracle
from oracle_pins import ALL_PINS, run_pin


@pytest.mark.parametrize("pin", ALL_PINS, ids=[p.__name__ for p in ALL_PINS])
def test_pin(pin):
    run_pin(pin, oracle)
