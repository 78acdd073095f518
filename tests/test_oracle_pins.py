"""The CPU oracle checked against library routines, closed forms, invariants
and brute force (no GPU).  The checks themselves live in ``oracle_pins.py``."""
import pytest

import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin()
