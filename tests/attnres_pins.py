"""Pins that tie the oracle's Attention Residuals aggregation to what its
definition fixes, independently of the oracle's own code.

"Kimi K3 technical FAQ", question "What does the architecture actually look
like?", and "Day-0 vLLM support for Kimi K3", section "Kimi K3's
architecture, and how vLLM serves it": logits of the earlier block outputs
against a learned pseudo-query, a softmax across them, the weighted sum, a
residual add and an output RMSNorm.  Read as, per token,

    p = softmax_m(scale <w, s_m>),  h = sum_m p_m s_m + x,
    y = h / sqrt(mean(h^2) + eps) * gamma.

The expected values use other routes: ``scipy.special.softmax``,
``np.einsum``, ``torch.nn.functional.rms_norm`` (fp64, CPU), closed forms
and invariants.  Mutated copies of the oracle must each fail one pin.
"""
from __future__ import annotations

import numpy as np

RTOL = 1e-12


def _close(a, b, rtol=RTOL, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} != {b.shape}"
    assert np.all(np.isfinite(a)), f"{what}: non-finite values"
    scale = max(1.0, float(np.max(np.abs(b)))) if b.size else 1.0
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert err <= rtol * scale, f"{what}: max abs err {err:.3e} > {rtol * scale:.3e}"


def _problem(seed, M, T, d):
    rng = np.random.default_rng(seed)
    f = lambda *s: rng.standard_normal(s).astype(np.float32)
    src = f(M, T, d)
    w = (rng.standard_normal(d) / np.sqrt(d) * 3).astype(np.float32)
    x = f(T, d)
    gamma = (1 + 0.2 * rng.standard_normal(d)).astype(np.float32)
    return src, w, x, gamma


def _rms_norm(h, gamma, eps):
    import torch
    ht = torch.from_numpy(np.asarray(h, dtype=np.float64))
    g = None if gamma is None else torch.from_numpy(np.asarray(gamma, dtype=np.float64))
    return torch.nn.functional.rms_norm(ht, (ht.shape[-1],), weight=g, eps=eps).numpy()


# A1 library route: logits by einsum, scipy's softmax, einsum aggregation,
#    torch's rms_norm; a logit scale other than 1 and eps not negligible
def pin_ar_library(O, M=5, T=7, d=48, scale=0.37, eps=0.3, seed=41):
    from scipy.special import softmax
    src, w, x, gamma = _problem(seed, M, T, d)
    s64 = src.astype(np.float64)
    p = softmax(scale * np.einsum("mtd,d->tm", s64, w.astype(np.float64)), axis=1)
    h_want = np.einsum("tm,mtd->td", p, s64) + x
    h, y = O.attnres(src, w, x=x, gamma=gamma, scale=scale, eps=eps)
    _close(h, h_want, what="h against einsum/scipy")
    _close(y, _rms_norm(h_want, gamma, eps), what="y against torch rms_norm")


# A2 a zero query weighs every source the same: h = mean of the sources + x
def pin_ar_zero_query(O, M=4, T=5, d=32, seed=42):
    src, w, x, gamma = _problem(seed, M, T, d)
    h, y = O.attnres(src, np.zeros_like(w), x=x, gamma=gamma, eps=1e-6)
    _close(h, src.astype(np.float64).mean(axis=0) + x, what="uniform weights")
    _close(y, _rms_norm(h, gamma, 1e-6), what="y")


# A3 one source: h = s + x exactly; no residual: h = s
def pin_ar_single_source(O, T=6, d=24, seed=43):
    src, w, x, gamma = _problem(seed, 1, T, d)
    h, _ = O.attnres(src, w, x=x)
    _close(h, src[0].astype(np.float64) + x, rtol=0.0, what="one source")
    h0, _ = O.attnres(src, w)
    _close(h0, src[0], rtol=0.0, what="one source, no residual")


# A4 a dominant logit selects its source (the others' weights ~ e^-300)
def pin_ar_dominant(O, M=6, T=4, d=16, seed=44):
    src, _, x, _ = _problem(seed, M, T, d)
    w = np.zeros(d, dtype=np.float32)
    w[0] = 1.0
    src[:, :, 0] = -1.0
    src[3, :, 0] = 1.0                       # source 3 has logit +scale, the rest -scale
    h, _ = O.attnres(src, w, x=x, scale=150.0)
    _close(h, src[3].astype(np.float64) + x, what="dominant source")


# A5 the order of the sources does not matter; without gamma, mean(y^2) is
#    ms / (ms + eps) with ms = mean(h^2)
def pin_ar_permutation_and_rms(O, M=5, T=6, d=40, seed=45):
    src, w, x, _ = _problem(seed, M, T, d)
    h, y = O.attnres(src, w, x=x, eps=0.05)
    perm = [3, 0, 4, 2, 1]
    hp, yp = O.attnres(src[perm], w, x=x, eps=0.05)
    _close(hp, h, rtol=1e-14, what="source order")
    _close(yp, y, rtol=1e-14, what="source order (y)")
    ms = (h * h).mean(axis=1)
    _close((y * y).mean(axis=1), ms / (ms + 0.05), what="mean square of y")


ALL_ATTNRES_PINS = [pin_ar_library, pin_ar_zero_query, pin_ar_single_source, pin_ar_dominant,
                    pin_ar_permutation_and_rms]
