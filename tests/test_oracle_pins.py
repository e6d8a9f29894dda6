"""The fp64 oracle against independent facts (CPU only)."""
import pytest

import oracle
from tests.oracle_pins import ALL_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=[p.__name__ for p in ALL_PINS])
def test_pin(pin):
    pin(oracle._load())
