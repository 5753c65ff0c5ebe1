"""The CPU oracle against its pins (see tests/oracle_pins.py)."""
import pytest

import oracle.method as M
from oracle_pins import PINS


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_oracle_pin(pin):
    pin(M)
