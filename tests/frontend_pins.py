"""Pins that tie the oracle's q/k front end to what its definition fixes,
independently of the oracle's own code.

"Kimi K3 technical FAQ", question "What is KDA, and why does a serving
engineer care?": queries and keys pass through a short convolution, Swish and
L2 normalisation.  Read as (channel c = h*dk + i, width W, tap W-1 on the
current token, inputs before a sequence's start taken from its convolution
state, oldest first, or zero):

    z_t[c] = sum_j w[c, j] x_{t-(W-1)+j}[c]
    a      = z * sigmoid(z)
    y_t[h] = a_t[h] / sqrt(|a_t[h]|^2 + eps)

and the new state of a sequence is its last W-1 inputs.

The expected values here are built with other routes: numpy's own
convolution (``np.convolve``), the tanh form of the logistic function
(sigmoid(z) = (1 + tanh(z/2)) / 2), ``np.linalg.norm``, and explicit history
arrays assembled by concatenation.  Each ``pin_*`` takes an
``oracle.Oracle`` handle and raises ``AssertionError`` on a mismatch;
mutated copies of the oracle must each fail one (``test_oracle_mutants.py``).
"""
from __future__ import annotations

import numpy as np

RTOL = 1e-12


def _swish(z):
    return z * 0.5 * (1.0 + np.tanh(0.5 * z))


def _normalise(a, eps):
    n = np.linalg.norm(a, axis=-1, keepdims=True)
    return a / np.sqrt(n * n + eps)


def _close(a, b, rtol=RTOL, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} != {b.shape}"
    assert np.all(np.isfinite(a)), f"{what}: non-finite values"
    scale = max(1.0, float(np.max(np.abs(b)))) if b.size else 1.0
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert err <= rtol * scale, f"{what}: max abs err {err:.3e} > {rtol * scale:.3e}"


def _problem(seed, lens, H, dk, W, with_state=True, slots=None, num_slots=None):
    """Random inputs for sequences of the given lengths (fp32 values)."""
    rng = np.random.default_rng(seed)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    T = int(cu[-1])
    x = rng.standard_normal((T, H, dk)).astype(np.float32)
    w = (rng.standard_normal((H * dk, W)) * 0.7).astype(np.float32)
    S = num_slots if num_slots is not None else len(lens)
    state = rng.standard_normal((S, W - 1, H, dk)).astype(np.float32) if with_state else None
    return x, w, cu, state


def _history(x, cu, b, state, slot, W):
    """[W-1 + L_b, H, dk]: the inputs preceding sequence b, then its own."""
    H, dk = x.shape[1:]
    pre = state[slot] if state is not None else np.zeros((W - 1, H, dk), np.float32)
    return np.concatenate([pre.astype(np.float64),
                           x[cu[b]:cu[b + 1]].astype(np.float64)], axis=0)


def _expected(x, w, cu, W, eps, state=None, slots=None):
    """y through np.convolve per channel, and the expected new state rows."""
    T, H, dk = x.shape
    y = np.zeros((T, H, dk))
    tails = {}
    for b in range(len(cu) - 1):
        slot = b if slots is None else int(slots[b])
        hist = _history(x, cu, b, state, slot, W)          # [W-1+L, H, dk]
        L = int(cu[b + 1] - cu[b])
        flat = hist.reshape(hist.shape[0], H * dk)
        z = np.zeros((L, H * dk))
        for c in range(H * dk if L > 0 else 0):
            # np.convolve flips its second operand: convolving with the taps
            # reversed gives sum_j w[c, j] hist[n + j, c]
            z[:, c] = np.convolve(flat[:, c], w[c, ::-1].astype(np.float64), mode="valid")
        a = _swish(z).reshape(L, H, dk)
        y[cu[b]:cu[b + 1]] = _normalise(a, eps)
        tails[slot] = hist[hist.shape[0] - (W - 1):] if W > 1 else hist[:0]
    return y, tails


# --------------------------------------------------------------------------
# F1  only the current-token tap, a per-channel gain g_c:  z = g_c x.
#     y = swish(g x) / sqrt(|swish(g x)|^2 + eps), eps not negligible.
def pin_fe_current_tap(O, H=3, dk=8, W=4, eps=0.37, seed=11):
    x, w, cu, state = _problem(seed, [5, 9], H, dk, W)
    gain = np.random.default_rng(seed + 1).uniform(0.5, 2.0, H * dk).astype(np.float32)
    w[:] = 0.0
    w[:, W - 1] = gain
    y, _ = O.qk_frontend(x, w, cu, W, eps, state=state)
    z = x.astype(np.float64) * gain.reshape(1, H, dk)
    _close(y, _normalise(_swish(z), eps), what="current-tap closed form")


# --------------------------------------------------------------------------
# F2  only the oldest tap: z_t = g_c x_{t-(W-1)}, the first W-1 outputs of
#     each sequence come from its own state rows, in order, through slots.
def pin_fe_oldest_tap(O, H=2, dk=4, W=4, eps=1e-3, seed=12):
    lens = [7, 2, 0, 5]
    slots = np.array([3, 0, 4, 1], dtype=np.int32)
    x, w, cu, state = _problem(seed, lens, H, dk, W, num_slots=5)
    gain = np.random.default_rng(seed + 1).uniform(0.5, 2.0, H * dk).astype(np.float32)
    w[:] = 0.0
    w[:, 0] = gain
    y, _ = O.qk_frontend(x, w, cu, W, eps, state=state, slots=slots)
    for b in range(len(lens)):
        hist = _history(x, cu, b, state, slots[b], W)
        shifted = hist[:lens[b]]                           # x_{t-(W-1)}
        want = _normalise(_swish(shifted * gain.reshape(1, H, dk)), eps)
        _close(y[cu[b]:cu[b + 1]], want, what=f"oldest tap, sequence {b}")


# --------------------------------------------------------------------------
# F3  general taps against np.convolve: several sequences, an empty one, two
#     shorter than W-1, a state through a slot permutation.
def pin_fe_convolve(O, H=3, dk=8, W=4, eps=1e-6, seed=13):
    lens = [1, 0, 12, 2, 30]
    slots = np.array([4, 2, 0, 5, 1], dtype=np.int32)
    x, w, cu, state = _problem(seed, lens, H, dk, W, num_slots=6)
    y, new_state = O.qk_frontend(x, w, cu, W, eps, state=state, slots=slots)
    want, tails = _expected(x, w, cu, W, eps, state, slots)
    _close(y, want, what="np.convolve route")
    for slot, rows in tails.items():
        _close(new_state[slot], rows, rtol=0.0, what=f"state rows of slot {slot}")
    untouched = 3
    _close(new_state[untouched], state[untouched], rtol=0.0, what="untouched slot")


# --------------------------------------------------------------------------
# F4  no state: history is zero; width 1 (no state at all) and width 8.
def pin_fe_zero_history(O, H=2, dk=16, eps=1e-6, seed=14):
    for W in (1, 2, 8):
        x, w, cu, _ = _problem(seed + W, [3, 11], H, dk, W, with_state=False)
        y, new_state = O.qk_frontend(x, w, cu, W, eps)
        want, tails = _expected(x, w, cu, W, eps)
        _close(y, want, what=f"zero history, W={W}")
        assert new_state.shape == (2, W - 1, H, dk)
        for slot, rows in tails.items():
            _close(new_state[slot], rows, rtol=0.0, what=f"W={W} state of slot {slot}")


# --------------------------------------------------------------------------
# F5  splitting a sequence and carrying the state across the split changes
#     nothing (the state is exactly the history the second part needs).
def pin_fe_chaining(O, H=2, dk=8, W=4, eps=1e-6, seed=15):
    x, w, cu, state = _problem(seed, [23], H, dk, W)
    y, s_full = O.qk_frontend(x, w, cu, W, eps, state=state)
    for cut in (0, 1, 2, 3, 10, 23):
        y1, s1 = O.qk_frontend(x[:cut], w, [0, cut], W, eps, state=state)
        y2, s2 = O.qk_frontend(x[cut:], w, [0, 23 - cut], W, eps, state=s1)
        _close(np.concatenate([y1, y2]), y, rtol=0.0, what=f"split at {cut}: outputs")
        _close(s2, s_full, rtol=0.0, what=f"split at {cut}: state")


# --------------------------------------------------------------------------
# F6  unit length: with eps far below |a|^2 every (token, head) row has norm 1.
def pin_fe_unit_rows(O, H=4, dk=32, W=4, seed=16):
    x, w, cu, state = _problem(seed, [40], H, dk, W)
    y, _ = O.qk_frontend(x, w, cu, W, 1e-30, state=state)
    n = np.linalg.norm(y, axis=-1)
    assert np.all(np.abs(n - 1.0) < 1e-13), f"row norms deviate by {np.max(np.abs(n - 1)):.2e}"


ALL_FRONTEND_PINS = [pin_fe_current_tap, pin_fe_oldest_tap, pin_fe_convolve,
                     pin_fe_zero_history, pin_fe_chaining, pin_fe_unit_rows]
