"""The oracle's q/k front end against what its definition fixes (library
convolution, closed forms, invariants); see ``frontend_pins.py``."""
import pytest

import frontend_pins


@pytest.mark.parametrize("pin", frontend_pins.ALL_FRONTEND_PINS, ids=lambda f: f.__name__)
def test_frontend_pin(oracle_lib, pin):
    pin(oracle_lib)


def test_frontend_rejects_bad_eps(oracle_lib):
    import numpy as np
    x = np.zeros((2, 1, 4), np.float32)
    with pytest.raises(ValueError):
        oracle_lib.qk_frontend(x, np.ones((4, 2), np.float32), [0, 2], 2, 0.0)


def test_frontend_zero_input_is_zero(oracle_lib):
    import numpy as np
    x = np.zeros((5, 2, 8), np.float32)
    y, st = oracle_lib.qk_frontend(x, np.ones((16, 4), np.float32), [0, 5], 4, 1e-6)
    assert np.array_equal(y, np.zeros_like(y)) and np.array_equal(st, np.zeros_like(st))
