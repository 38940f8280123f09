"""The fp64 oracle checked against hand-worked values, exact rational brute force,
closed forms, library routines and independent reformulations (see oracle_pins.py)."""
import pytest

import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(oracle_lib, pin):
    pin()
