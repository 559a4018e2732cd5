"""The CPU oracle against its pins: worked examples, closed forms, invariants,
brute force, and library routines (see ``pins.py``)."""
import pytest

import oracle
import pins


@pytest.fixture(scope="module")
def O():
    return oracle.default()


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=[p.__name__ for p in pins.ALL_PINS])
def test_pin(O, pin):
    pin(O)
