"""The CPU oracle against its pins (library routines, format constants, brute force,
closed forms, invariants the pages fix).  No GPU needed."""
import pytest

from tests import oracle_pins as P


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()
