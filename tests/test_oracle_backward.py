"""The oracle's backward pass against its pins (CPU)."""
import pytest

import oracle
from oracle_backward_pins import BACKWARD_PINS


@pytest.mark.parametrize("pin", BACKWARD_PINS, ids=[p.__name__ for p in BACKWARD_PINS])
def test_backward_pin(pin):
    pin(oracle.load())
