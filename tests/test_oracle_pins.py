"""The fp64 oracle against its pins (closed forms, invariants, the masked-attention
formulation, library reductions).  CPU only."""
import pytest

import oracle
from oracle_pins import PINS


@pytest.fixture(scope="module")
def lib():
    return oracle.load()


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(lib, pin):
    pin(lib)
