"""The oracle against brute force, closed forms, invariants and library routines."""
import pytest

import oracle.block as ob
from oracle_pins import ALL_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(ob)
