"""The CPU oracle against hand-worked examples, closed forms, independent
library routines, brute force and the method's invariants."""
import pytest

import oracle
from tests.oracle_pins import ALL_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=[p.__name__ for p in ALL_PINS])
def test_pin(pin):
    pin(oracle)
