"""The chunked prefill decomposition, pinned to the oracle on the CPU.

``chunked_model`` restates in fp64 numpy the algebra the prefill kernels
evaluate (the Gram matrices A and B blockwise around a reference row, the
UT transform T = (I + A)^-1, W, M, Q', U~, O~, Kd and the three products with
the state per chunk).  In exact arithmetic it must equal the token-by-token
oracle to rounding (1e-12 here); with the kernels' rounding points emulated
it must stay inside the 2e-3 parity bar in every regime, including the
exact-write regime (alpha = 1, beta = 1, q = k) where the output is formed
by cancellation.  The last tests keep the reason for each rounding choice
measurable: the earlier, cheaper choices break the bar in the regime named.
"""
import numpy as np
import pytest

import chunked_model as cm
from parity import TOL, seq_head_err, state_err


def _inputs(lens, H, d, seed, shift=2.0, beta_shift=0.0, state_std=0.05, bf16=True):
    rng = np.random.default_rng(seed)
    T = int(sum(lens))

    def unit(x):
        return x / np.linalg.norm(x, axis=-1, keepdims=True)

    q = unit(rng.standard_normal((T, H, d))).astype(np.float32)
    k = unit(rng.standard_normal((T, H, d))).astype(np.float32)
    v = rng.standard_normal((T, H, d)).astype(np.float32)
    if bf16:
        q, k, v = (cm.to_bf16(x).astype(np.float32) for x in (q, k, v))
    beta = (1.0 / (1.0 + np.exp(-(rng.standard_normal((T, H)) + beta_shift)))).astype(np.float32)
    g = (-np.logaddexp(0.0, rng.standard_normal((T, H, d)) + shift)).astype(np.float32)
    init = (state_std * rng.standard_normal((len(lens), H, d, d))).astype(np.float32)
    cu = np.cumsum([0] + list(lens)).astype(np.int32)
    return q, k, v, g, beta, cu, init


def _exact_write(lens, H, d, seed):
    rng = np.random.default_rng(seed)
    T = int(sum(lens))
    k = rng.standard_normal((T, H, d))
    k = (k / np.linalg.norm(k, axis=-1, keepdims=True)).astype(np.float32)
    v = rng.standard_normal((T, H, d)).astype(np.float32)
    g = np.zeros((T, H, d), np.float32)
    beta = np.ones((T, H), np.float32)
    init = (0.02 * rng.standard_normal((len(lens), H, d, d))).astype(np.float32)
    cu = np.cumsum([0] + list(lens)).astype(np.int32)
    return k, k, v, g, beta, cu, init


def _errs(args, interval, rnd, oracle_lib):
    q, k, v, g, beta, cu, init = args
    ro, rf, rs = oracle_lib.prefill(q, k, v, g, beta, cu, initial_state=init,
                                    snapshot_interval=interval)
    mo, mf, ms = cm.prefill(q, k, v, g, beta, cu, initial_state=init,
                            snapshot_interval=interval, rnd=rnd)
    es = state_err(ms, rs) if rs.shape[0] else 0.0
    return seq_head_err(mo, ro, cu), state_err(mf, rf), es


@pytest.mark.parametrize("d", [16, 64])
@pytest.mark.parametrize("shift", [2.0, -4.0, 0.0])
def test_exact_decomposition_equals_oracle(d, shift, oracle_lib):
    """Ragged and empty sequences, initial states, snapshots every 64 tokens:
    the decomposition is the recurrence (fp64 rounding only)."""
    args = _inputs([200, 64, 1, 97, 0, 130], H=2, d=d, seed=int(10 * d - shift), shift=shift)
    eo, ef, es = _errs(args, 64, cm.EXACT, oracle_lib)
    assert eo < 1e-12 and ef < 1e-12 and es < 1e-12, (eo, ef, es)


def test_exact_decomposition_special_cases(oracle_lib):
    """beta = 0 (pure decay), exact write (alpha = beta = 1, q = k) and
    near-total forgetting bursts (the Gram factors then span e^+-240 inside a
    16-row block, inside fp64's range)."""
    q, k, v, g, beta, cu, init = _inputs([150, 77], H=2, d=32, seed=5)
    assert max(_errs((q, k, v, g, np.zeros_like(beta), cu, init), 64, cm.EXACT,
                     oracle_lib)) < 1e-12
    assert max(_errs(_exact_write([130, 70], 2, 32, 6), 0, cm.EXACT, oracle_lib)) < 1e-12
    g = g.copy()
    g[40:52, 1, :] = -30.0
    g[:, :, ::3] = -12.0
    assert max(_errs((q, k, v, g, beta, cu, init), 64, cm.EXACT, oracle_lib)) < 1e-11


@pytest.mark.parametrize("d", [16, 128])
def test_kernel_rounding_exact_write(d, oracle_lib):
    """The kernels' rounding points in the exact-write regime: the output is
    formed by cancellation (M = B TB = I when q = k and beta = 1), and stays
    far inside the bar; the state carries fp16-level rounding."""
    eo, ef, _ = _errs(_exact_write([200, 64, 137, 1], 2, d, 21 + d), 0, cm.kernel_rounding(),
                      oracle_lib)
    assert eo <= 1e-4 and ef <= 1e-3, (eo, ef)


@pytest.mark.parametrize("shift", [2.0, -2.0, -5.0, -20.0])
def test_kernel_rounding_decay_regimes(shift, oracle_lib):
    """The kernels' rounding points across decay strengths, down to no
    forgetting with beta ~ 1 (shift -20, beta_shift 4)."""
    bs = 4.0 if shift == -20.0 else 0.0
    args = _inputs([512], H=2, d=128, seed=7, shift=shift, beta_shift=bs, state_std=0.02)
    eo, ef, es = _errs(args, 128, cm.kernel_rounding(), oracle_lib)
    assert max(eo, ef, es) <= 5e-4, (eo, ef, es)


def test_single_bf16_gram_and_key_operands_break_exact_write(oracle_lib):
    """One bf16 rounding of K e^G (in W and Q') and of the diagonal A blocks
    misses the bar at d = 16 in the exact-write regime: A and B then round
    differently and M = B TB drifts from I by ~1e-3."""
    args = _exact_write([200, 64, 137, 1], 2, 16, 37)
    eo, ef, _ = _errs(args, 0, cm.kernel_rounding(ktilde="bf16", diag_a="bf16"), oracle_lib)
    assert eo > TOL, eo
    eo2, _, _ = _errs(args, 0, cm.kernel_rounding(), oracle_lib)
    assert eo2 < eo / 50, (eo2, eo)


def test_single_bf16_scan_operands_break_the_bar(oracle_lib):
    """W, Q' and Kd as single bf16 values (no per-tile fp16 exponent) miss the
    bar under weak decay; fp16 with a power-of-two exponent per tile stays
    at a few 1e-4."""
    args = _inputs([512], H=2, d=128, seed=7, shift=-5.0, state_std=0.02)
    bf = max(_errs(args, 128, cm.kernel_rounding(scan_ops="bf16"), oracle_lib))
    f16 = max(_errs(args, 128, cm.kernel_rounding(), oracle_lib))
    assert bf > TOL and f16 < 5e-4, (bf, f16)
