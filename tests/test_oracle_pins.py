"""The fp64 oracle against its pins (pages' numbers, closed forms, exact
rationals, library routines, brute force)."""
import pytest

import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(orc, pin):
    pin(orc)
