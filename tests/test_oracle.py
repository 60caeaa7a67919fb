"""The CPU oracle against closed forms, invariants, library routines, finite
differences and the hand-worked fixture (no GPU)."""
import pytest

import oracle
from oracle_pins import ALL_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=[p.__name__ for p in ALL_PINS])
def test_oracle_pin(pin):
    pin(oracle.flp_oracle)
