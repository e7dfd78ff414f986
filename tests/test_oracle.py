"""The CPU oracle against its pins (no GPU)."""
import pytest

import oracle
from tests.oracle_pins import PINS


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_oracle_pin(pin):
    pin(oracle)
