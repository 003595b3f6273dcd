"""The fp64 oracle against what the definition of the recurrence fixes
(closed forms, invariants, brute force); see ``oracle_pins.py``."""
import pytest

import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(oracle_lib, pin):
    pin(oracle_lib)


def test_exact_write_d128(oracle_lib):
    oracle_pins.pin_exact_write(oracle_lib, dk=128, dv=128, T=12, H=1)


def test_product_form_d16(oracle_lib):
    oracle_pins.pin_product_form(oracle_lib, dk=16, dv=16, T=8, H=1, seed=3)


def test_default_scale(oracle_lib):
    import numpy as np
    rng = np.random.default_rng(5)
    T, H, dk, dv = 6, 1, 9, 4
    q, k, v, g, beta = oracle_pins._rand_problem(rng, T, H, dk, dv)
    o_default, _, _ = oracle_lib.prefill(q, k, v, g, beta, [0, T])
    o_one, _, _ = oracle_lib.prefill(q, k, v, g, beta, [0, T], scale=1.0)
    assert np.array_equal(o_default, o_one * (1.0 / np.sqrt(dk))) or \
        np.allclose(o_default, o_one / np.sqrt(dk), rtol=1e-15, atol=0)


def test_state_size_independent_of_length(oracle_lib):
    import numpy as np
    rng = np.random.default_rng(6)
    for T in (1, 17, 200):
        q, k, v, g, beta = oracle_pins._rand_problem(rng, T, 2, 4, 3)
        _, final, _ = oracle_lib.prefill(q, k, v, g, beta, [0, T])
        assert final.shape == (1, 2, 4, 3)


def test_empty_sequence_keeps_initial_state(oracle_lib):
    import numpy as np
    rng = np.random.default_rng(7)
    q, k, v, g, beta = oracle_pins._rand_problem(rng, 3, 1, 4, 3)
    S0 = rng.standard_normal((2, 1, 4, 3))
    out, final, _ = oracle_lib.prefill(q, k, v, g, beta, [0, 0, 3],
                                       initial_state=S0)
    assert np.array_equal(final[0], S0[0])
