"""The oracle's Attention Residuals aggregation against library routes,
closed forms and invariants; see ``attnres_pins.py``."""
import pytest

import attnres_pins


@pytest.mark.parametrize("pin", attnres_pins.ALL_ATTNRES_PINS, ids=lambda f: f.__name__)
def test_attnres_pin(oracle_lib, pin):
    pin(oracle_lib)
