"""The CPU oracle against its pins (brute force, library routines, closed
forms, invariants).  No GPU involved."""
import pytest

from pins import ALL_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=[p.__name__ for p in ALL_PINS])
def test_pin(pin):
    pin()
