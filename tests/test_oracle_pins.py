"""The fp64 oracle against its pins (closed forms, hand formulas, invariants,
independent library implementations, finite differences, high precision)."""
import pytest

import oracle
from tests.oracle_pins import PINS


@pytest.fixture(scope="module")
def orc():
    return oracle.default()


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(orc, pin):
    pin(orc)
