"""The float64 oracle against facts fixed by the mathematics (tests/pins.py)."""
import pytest

import oracle
from pins import ALL_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda p: p.__name__)
def test_oracle_pin(pin):
    pin(oracle)
