"""The CPU oracle against closed forms, invariants, brute force and the
pages' printed byte counts (each pin is documented in tests/pins.py)."""
import pytest

import pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(orc, pin):
    pin(orc)
