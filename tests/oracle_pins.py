"""Pins that tie the fp64 oracle to what the definition of the KDA recurrence
fixes, independently of the oracle's own code.

Each ``pin_*`` function takes an ``oracle.Oracle`` handle and raises
``AssertionError`` when the handle's results break the pinned fact.  The
real oracle must pass all of them (``test_oracle_pins.py``); deliberately
mutated copies of the oracle must each fail at least one
(``test_oracle_mutants.py``).

The recurrence pinned (read from "Kimi K3 technical FAQ", question "What is
KDA, and why does a serving engineer care?": delta rule with a per-channel
forget gate and a dk x dv state per head):

    S_t = (I - b_t k_t k_t^T) Diag(a_t) S_{t-1} + b_t k_t v_t^T,
    o_t = dk^-1/2 S_t^T q_t,   a_t = exp(g_t).

The pages print no worked example, so every pin is a closed form, an
invariant or an independent brute-force evaluation of that definition.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

RTOL = 1e-12


def _rng(seed):
    return np.random.default_rng(seed)


def _unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _rand_problem(rng, T, H, dk, dv, unit_keys=True, g_scale=1.0):
    q = rng.standard_normal((T, H, dk))
    k = rng.standard_normal((T, H, dk))
    if unit_keys:
        q, k = _unit(q), _unit(k)
    v = rng.standard_normal((T, H, dv))
    g = -np.log1p(np.exp(rng.standard_normal((T, H, dk)))) * g_scale
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((T, H))))
    f32 = lambda a: a.astype(np.float32)
    return f32(q), f32(k), f32(v), f32(g), f32(beta)


def _close(a, b, rtol=RTOL, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert np.all(np.isfinite(a)), f"{what}: non-finite values"
    scale = max(1.0, float(np.max(np.abs(b)))) if b.size else 1.0
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert err <= rtol * scale, f"{what}: max abs err {err:.3e} > {rtol * scale:.3e}"


# --------------------------------------------------------------------------
# P1  exact write: alpha = 1, beta = 1, |k_t| = 1  =>  S_t^T k_t = v_t.
#     With q_t = k_t the output is dk^-1/2 v_t, whatever S_{t-1} was.
# --------------------------------------------------------------------------
def pin_exact_write(O, dk=16, dv=16, T=24, H=2, seed=11):
    rng = _rng(seed)
    # keys with entries +-1/4 in 16 channels have |k| = 1 exactly in binary
    k = np.zeros((T, H, dk))
    for t in range(T):
        for h in range(H):
            idx = rng.choice(dk, size=16, replace=False)
            k[t, h, idx] = rng.choice([-0.25, 0.25], size=16)
    v = rng.standard_normal((T, H, dv))
    g = np.zeros((T, H, dk))
    beta = np.ones((T, H))
    S0 = rng.standard_normal((1, H, dk, dv))
    out, final, _ = O.prefill(k, k, v, g, beta, [0, T], initial_state=S0)
    v32 = v.astype(np.float32).astype(np.float64)
    _close(out * np.sqrt(dk), v32, 1e-12, "P1 o_t = dk^-1/2 v_t")
    # the last write is recalled exactly from the final state
    recall = np.einsum("hij,hi->hj", final[0], k[-1])
    _close(recall, v32[-1], 1e-12, "P1 S_T^T k_T = v_T")


# --------------------------------------------------------------------------
# P2  beta = 0: pure channel decay, S_t = Diag(exp(sum_{s<=t} g_s)) S_0.
# --------------------------------------------------------------------------
def pin_beta_zero(O, dk=8, dv=6, T=40, H=3, seed=12):
    rng = _rng(seed)
    q, k, v, g, _ = _rand_problem(rng, T, H, dk, dv, g_scale=0.3)
    beta = np.zeros((T, H), dtype=np.float32)
    S0 = rng.standard_normal((1, H, dk, dv))
    out, final, _ = O.prefill(q, k, v, g, beta, [0, T], initial_state=S0)
    G = np.cumsum(g.astype(np.float64), axis=0)           # [T, H, dk]
    S_t = np.exp(G)[..., None] * S0[0][None]              # [T, H, dk, dv]
    o_ref = np.einsum("thij,thi->thj", S_t, q.astype(np.float64)) / np.sqrt(dk)
    _close(out, o_ref, 1e-12, "P2 outputs")
    _close(final[0], S_t[-1], 1e-12, "P2 final state")


# --------------------------------------------------------------------------
# P3  split / resume: running [0, L) whole equals running [0, m) and then
#     [m, L) from the fp64 state at m, bit for bit; snapshot j equals the
#     final state of the first j*interval tokens.
# --------------------------------------------------------------------------
def pin_split_resume(O, dk=8, dv=8, T=50, H=2, m=23, interval=10, seed=13):
    rng = _rng(seed)
    q, k, v, g, beta = _rand_problem(rng, T, H, dk, dv)
    S0 = rng.standard_normal((1, H, dk, dv))
    out, final, snaps = O.prefill(q, k, v, g, beta, [0, T], initial_state=S0,
                                  snapshot_interval=interval)
    o1, s1, _ = O.prefill(q[:m], k[:m], v[:m], g[:m], beta[:m], [0, m],
                          initial_state=S0)
    o2, s2, _ = O.prefill(q[m:], k[m:], v[m:], g[m:], beta[m:], [0, T - m],
                          initial_state=s1)
    assert np.array_equal(np.concatenate([o1, o2]), out), "P3 resumed outputs differ"
    assert np.array_equal(s2, final), "P3 resumed final state differs"
    assert snaps.shape[0] == T // interval, "P3 snapshot count"
    for j in range(1, T // interval + 1):
        L = j * interval
        _, sj, _ = O.prefill(q[:L], k[:L], v[:L], g[:L], beta[:L], [0, L],
                             initial_state=S0)
        assert np.array_equal(snaps[j - 1], sj[0]), f"P3 snapshot {j}"


# --------------------------------------------------------------------------
# P4  brute force of the literal product form on T <= 8 tokens:
#     M_t = (I - b_t k_t k_t^T) Diag(a_t),
#     S_t = (M_t ... M_1) S_0 + sum_{s<=t} (M_t ... M_{s+1}) b_s k_s v_s^T.
#     Non-unit keys, random gates; dense dk x dk matrices, no recursion.
# --------------------------------------------------------------------------
def _product_form(q, k, v, g, beta, S0, scale):
    T, dk = k.shape
    M = [(np.eye(dk) - beta[t] * np.outer(k[t], k[t])) @ np.diag(np.exp(g[t]))
         for t in range(T)]

    def chain(hi, lo):  # M_hi ... M_lo (1-based, empty product = I)
        P = np.eye(dk)
        for r in range(lo, hi + 1):
            P = M[r - 1] @ P
        return P

    outs, S = [], None
    for t in range(1, T + 1):
        S = chain(t, 1) @ S0
        for s in range(1, t + 1):
            S = S + chain(t, s + 1) @ (beta[s - 1] * np.outer(k[s - 1], v[s - 1]))
        outs.append(scale * S.T @ q[t - 1])
    return np.array(outs), S


def pin_product_form(O, dk=5, dv=4, T=8, H=2, seed=14):
    rng = _rng(seed)
    q, k, v, g, beta = _rand_problem(rng, T, H, dk, dv, unit_keys=False)
    S0 = rng.standard_normal((1, H, dk, dv))
    out, final, _ = O.prefill(q, k, v, g, beta, [0, T], initial_state=S0)
    f = lambda a: a.astype(np.float64)
    for h in range(H):
        o_ref, s_ref = _product_form(f(q[:, h]), f(k[:, h]), f(v[:, h]),
                                     f(g[:, h]), f(beta[:, h]), S0[0, h],
                                     1.0 / np.sqrt(dk))
        _close(out[:, h], o_ref, 1e-12, f"P4 outputs head {h}")
        _close(final[0, h], s_ref, 1e-12, f"P4 final state head {h}")


def pin_exact_rational(O):
    """P4 in exact rational arithmetic on a 2x2 state, 3 tokens.  Keys,
    values, queries, betas and the initial state are exact binary fractions;
    each gate is the fp64 exp of an fp32 log-gate, taken as an exact
    rational, so the only rounding left is the oracle's own fp64 work."""
    dk = dv = 2
    F = Fraction
    k = [[F(1, 2), F(-1, 4)], [F(3, 4), F(1, 2)], [F(-1, 2), F(1, 1)]]
    q = [[F(1, 1), F(0)], [F(1, 4), F(-1, 2)], [F(3, 4), F(1, 4)]]
    v = [[F(2), F(-1)], [F(1, 2), F(3, 2)], [F(-3, 4), F(1, 4)]]
    g32 = np.log(np.array([[0.5, 1.0], [0.25, 0.5], [1.0, 0.25]])).astype(np.float32)
    alpha = [[F(float(np.exp(np.float64(x)))) for x in row] for row in g32]
    beta = [F(1, 2), F(3, 4), F(1, 4)]
    S = [[F(1, 8), F(-1, 4)], [F(1, 2), F(3, 8)]]
    toarr = lambda x: np.array(x, dtype=np.float64)
    S0 = toarr(S)[None, None]
    outs = []
    for t in range(3):
        # (I - b k k^T) Diag(a) S + b k v^T in exact arithmetic
        DS = [[alpha[t][i] * S[i][j] for j in range(dv)] for i in range(dk)]
        P = [[(1 if i == r else 0) - beta[t] * k[t][i] * k[t][r]
              for r in range(dk)] for i in range(dk)]
        S = [[sum(P[i][r] * DS[r][j] for r in range(dk)) + beta[t] * k[t][i] * v[t][j]
              for j in range(dv)] for i in range(dk)]
        outs.append([sum(q[t][i] * S[i][j] for i in range(dk)) for j in range(dv)])
    out, final, _ = O.prefill(toarr(q)[:, None], toarr(k)[:, None],
                              toarr(v)[:, None], g32[:, None],
                              toarr(beta)[:, None], [0, 3], initial_state=S0,
                              scale=1.0)
    _close(out[:, 0], toarr(outs), 1e-14, "exact rational outputs")
    _close(final[0, 0], toarr(S), 1e-14, "exact rational state")


# --------------------------------------------------------------------------
# P5  orthonormal-key recall: alpha = 1, beta = 1, k_t = e_t  =>  after dk
#     writes, row t of S equals v_t (non-interfering keys are exact).
# --------------------------------------------------------------------------
def pin_orthonormal_recall(O, dk=12, dv=7, H=2, seed=15):
    rng = _rng(seed)
    T = dk
    k = np.zeros((T, H, dk))
    for t in range(T):
        k[t, :, t] = 1.0
    q = _unit(rng.standard_normal((T, H, dk)))
    v = rng.standard_normal((T, H, dv))
    g = np.zeros((T, H, dk))
    beta = np.ones((T, H))
    S0 = rng.standard_normal((1, H, dk, dv))
    _, final, _ = O.prefill(q, k, v, g, beta, [0, T], initial_state=S0)
    _close(final[0], np.transpose(v.astype(np.float32).astype(np.float64),
                                  (1, 0, 2)), 1e-13, "P5 recall")


# --------------------------------------------------------------------------
# P6  dk = 1: s_t = (1 - b_t k_t^2) a_t s_{t-1} + b_t k_t v_t, a first-order
#     linear IIR filter per value column.  Constant coefficients are checked
#     against scipy.signal.lfilter, varying ones against the closed-form
#     product-sum  s_T = P_T s_0 + sum_t (prod_{r>t} c_r) b_t k_t v_t.
# --------------------------------------------------------------------------
def pin_scalar_iir(O, dv=5, T=30, seed=16):
    from scipy.signal import lfilter
    rng = _rng(seed)
    a, b, kk = 0.75, 0.5, 0.625       # alpha, beta, key: exact in binary
    v = rng.standard_normal((T, 1, dv)).astype(np.float32)
    q = np.full((T, 1, 1), 0.875, dtype=np.float32)
    k = np.full((T, 1, 1), kk, dtype=np.float32)
    g = np.full((T, 1, 1), np.log(a), dtype=np.float32)
    beta = np.full((T, 1), b, dtype=np.float32)
    s0 = rng.standard_normal((1, 1, 1, dv))
    out, final, _ = O.prefill(q, k, v, g, beta, [0, T], initial_state=s0,
                              scale=1.0)
    a_eff = float(np.exp(np.float64(np.float32(np.log(a)))))
    c = (1.0 - b * kk * kk) * a_eff
    y = lfilter([b * kk], [1.0, -c], v[:, 0, :].astype(np.float64), axis=0,
                zi=(c * s0[0, 0, 0])[None, :])[0]
    _close(out[:, 0, :], 0.875 * y, 1e-12, "P6 lfilter outputs")
    _close(final[0, 0, 0], y[-1], 1e-12, "P6 lfilter state")
    # time-varying coefficients: closed-form product-sum
    g2 = -np.log1p(np.exp(rng.standard_normal((T, 1, 1)))).astype(np.float32)
    beta2 = (1 / (1 + np.exp(-rng.standard_normal((T, 1))))).astype(np.float32)
    k2 = rng.uniform(-1, 1, (T, 1, 1)).astype(np.float32)
    _, final2, _ = O.prefill(q, k2, v, g2, beta2, [0, T], initial_state=s0)
    f = lambda x: x.astype(np.float64).reshape(T)
    cs = (1 - f(beta2) * f(k2) ** 2) * np.exp(f(g2))
    tail = np.array([np.prod(cs[t + 1:]) for t in range(T)])
    ref = np.prod(cs) * s0[0, 0, 0] + np.sum(
        (tail * f(beta2) * f(k2))[:, None] * v[:, 0, :].astype(np.float64), axis=0)
    _close(final2[0, 0, 0], ref, 1e-12, "P6 product-sum state")


# --------------------------------------------------------------------------
# P7  linearity: outputs and states are jointly linear in (v, S_0) for fixed
#     q, k, g, beta.
# --------------------------------------------------------------------------
def pin_linearity(O, dk=6, dv=5, T=30, H=2, seed=17):
    rng = _rng(seed)
    q, k, v1, g, beta = _rand_problem(rng, T, H, dk, dv)
    v2 = rng.standard_normal((T, H, dv)).astype(np.float32)
    A = rng.standard_normal((1, H, dk, dv))
    B = rng.standard_normal((1, H, dk, dv))
    c = 0.5  # a power of two: scaling by it is exact in binary
    o1, s1, _ = O.prefill(q, k, v1, g, beta, [0, T], initial_state=A)
    o2, s2, _ = O.prefill(q, k, v2, g, beta, [0, T], initial_state=B)
    # superposition of exact inputs: (v1, A) = (v1, 0) + (0, A)
    o4, s4, _ = O.prefill(q, k, np.zeros_like(v1), g, beta, [0, T],
                          initial_state=A)
    o5, s5, _ = O.prefill(q, k, v1, g, beta, [0, T],
                          initial_state=np.zeros_like(A))
    _close(o4 + o5, o1, 1e-12, "P7 outputs (superposition)")
    _close(s4 + s5, s1, 1e-12, "P7 states (superposition)")
    # homogeneity with an exact factor: (c v2, c B) = c (v2, B)
    o3, s3, _ = O.prefill(q, k, (c * v2).astype(np.float32), g, beta, [0, T],
                          initial_state=c * B)
    _close(o3, c * o2, 1e-13, "P7 outputs (scaling)")
    _close(s3, c * s2, 1e-13, "P7 states (scaling)")


# --------------------------------------------------------------------------
# P8  contraction bound: |k| <= 1, alpha <= 1, beta in [0,1]
#     =>  ||S_t||_F <= ||S_{t-1}||_F + beta_t ||v_t||.
# --------------------------------------------------------------------------
def pin_contraction(O, dk=8, dv=8, T=60, H=2, seed=18):
    rng = _rng(seed)
    q, k, v, g, beta = _rand_problem(rng, T, H, dk, dv)
    k = (k * rng.uniform(0.3, 1.0, (T, H, 1))).astype(np.float32)
    S0 = 3.0 * rng.standard_normal((1, H, dk, dv))
    _, _, snaps = O.prefill(q, k, v, g, beta, [0, T], initial_state=S0,
                            snapshot_interval=1)
    norms = np.linalg.norm(snaps, axis=(2, 3))          # [T, H]
    prev = np.concatenate([np.linalg.norm(S0, axis=(2, 3)), norms[:-1]])
    bound = prev + beta.astype(np.float64) * np.linalg.norm(v.astype(np.float64), axis=2)
    assert np.all(norms <= bound * (1 + 1e-12)), "P8 contraction bound violated"


# --------------------------------------------------------------------------
# P9  dv-permutation equivariance: permuting the columns of v and S_0
#     permutes the columns of o and S (value columns evolve independently).
# --------------------------------------------------------------------------
def pin_permutation(O, dk=6, dv=9, T=25, H=2, seed=19):
    rng = _rng(seed)
    q, k, v, g, beta = _rand_problem(rng, T, H, dk, dv)
    S0 = rng.standard_normal((1, H, dk, dv))
    perm = rng.permutation(dv)
    o1, s1, _ = O.prefill(q, k, v, g, beta, [0, T], initial_state=S0)
    o2, s2, _ = O.prefill(q, k, v[..., perm], g, beta, [0, T],
                          initial_state=S0[..., perm])
    assert np.array_equal(o1[..., perm], o2), "P9 output columns"
    assert np.array_equal(s1[..., perm], s2), "P9 state columns"


# --------------------------------------------------------------------------
# P10 alpha = 1, beta = 0: the state never changes and o_t = dk^-1/2 S_0^T q_t.
# --------------------------------------------------------------------------
def pin_frozen_state(O, dk=10, dv=7, T=15, H=2, seed=20):
    rng = _rng(seed)
    q, k, v, _, _ = _rand_problem(rng, T, H, dk, dv)
    g = np.zeros((T, H, dk), dtype=np.float32)
    beta = np.zeros((T, H), dtype=np.float32)
    S0 = rng.standard_normal((1, H, dk, dv))
    out, final, _ = O.prefill(q, k, v, g, beta, [0, T], initial_state=S0)
    ref = np.einsum("hij,thi->thj", S0[0], q.astype(np.float64)) / np.sqrt(dk)
    _close(out, ref, 1e-13, "P10 outputs")
    assert np.array_equal(final, S0), "P10 state must not change"


# --------------------------------------------------------------------------
# Packing: each sequence of a varlen batch runs from its own initial state;
# the packed run equals separate runs, and snapshots land per sequence.
# --------------------------------------------------------------------------
def pin_varlen_packing(O, dk=6, dv=5, H=3, seed=21, interval=4):
    rng = _rng(seed)
    lens = [7, 0, 12, 4, 1]
    T = sum(lens)
    q, k, v, g, beta = _rand_problem(rng, T, H, dk, dv)
    S0 = rng.standard_normal((len(lens), H, dk, dv))
    cu = np.concatenate([[0], np.cumsum(lens)])
    out, final, snaps = O.prefill(q, k, v, g, beta, cu, initial_state=S0,
                                  snapshot_interval=interval)
    row = 0
    for b, L in enumerate(lens):
        s, e = cu[b], cu[b + 1]
        o_b, f_b, sn_b = O.prefill(q[s:e], k[s:e], v[s:e], g[s:e], beta[s:e],
                                   [0, L], initial_state=S0[b:b + 1],
                                   snapshot_interval=interval)
        assert np.array_equal(o_b, out[s:e]), f"packing outputs seq {b}"
        assert np.array_equal(f_b[0], final[b]), f"packing final seq {b}"
        n = L // interval
        assert np.array_equal(sn_b, snaps[row:row + n]), f"packing snaps seq {b}"
        row += n
    assert row == snaps.shape[0]


# --------------------------------------------------------------------------
# Decode = prefill: T chained single-token decode steps equal one prefill of
# length T (the same recurrence); slots remap which state row is used.
# --------------------------------------------------------------------------
def pin_decode_matches_prefill(O, dk=8, dv=6, T=20, N=3, H=2, seed=22):
    rng = _rng(seed)
    q, k, v, g, beta = _rand_problem(rng, T * N, H, dk, dv)
    shp = lambda a: a.reshape(T, N, *a.shape[1:])
    S0 = rng.standard_normal((N, H, dk, dv))
    slots = np.array([2, 0, 1], dtype=np.int32)
    state = np.zeros((N, H, dk, dv))
    state[slots] = S0
    out_d, st = O.decode(shp(q), shp(k), shp(v), shp(g), shp(beta), state,
                         slots=slots)
    for n in range(N):
        sel = lambda a: shp(a)[:, n]
        o_p, f_p, _ = O.prefill(sel(q), sel(k), sel(v), sel(g), sel(beta),
                                [0, T], initial_state=S0[n:n + 1])
        assert np.array_equal(out_d[:, n], o_p), f"decode outputs seq {n}"
        assert np.array_equal(st[slots[n]], f_p[0]), f"decode state seq {n}"


# --------------------------------------------------------------------------
# P11 absolute snapshot positions ("Day-0 vLLM support for Kimi K3", section
#     "Kimi K3's architecture, and how vLLM serves it": snapshots at block
#     boundaries, the prefix-match granularity independent of where a call
#     starts).  A sequence whose first token sits at absolute position s gets
#     a snapshot at every multiple P of the interval in (s, s + L]; it must be
#     the final state of a separate run over the sequence's first P - s
#     tokens, the count is sum floor((s + L) / I) - floor(s / I), rows come in
#     sequence order, and start positions of 0 change nothing.
def pin_absolute_snapshots(O, dk=5, dv=4, H=2, seed=23, interval=5):
    rng = _rng(seed)
    lens = [4, 0, 13, 9, 7]
    starts = [3, 10, 12, 0, 6]      # 3 + 4 reaches 5; 10 + 0 takes nothing; ...
    cu = np.concatenate([[0], np.cumsum(lens)])
    T = int(cu[-1])
    q, k, v, g, beta = _rand_problem(rng, T, H, dk, dv)
    S0 = rng.standard_normal((len(lens), H, dk, dv))
    _, final, snaps = O.prefill(q, k, v, g, beta, cu, initial_state=S0,
                                snapshot_interval=interval, start_pos=starts)
    want_count = sum((s + L) // interval - s // interval for s, L in zip(starts, lens))
    assert snaps.shape[0] == want_count, f"{snaps.shape[0]} snapshots, expected {want_count}"
    row = 0
    for b, (s, L) in enumerate(zip(starts, lens)):
        a, e = int(cu[b]), int(cu[b + 1])
        for P in range((s // interval + 1) * interval, s + L + 1, interval):
            m = P - s
            _, sm, _ = O.prefill(q[a:a + m], k[a:a + m], v[a:a + m], g[a:a + m],
                                 beta[a:a + m], [0, m], initial_state=S0[b:b + 1])
            _close(snaps[row], sm[0], what=f"snapshot at absolute {P} of sequence {b}")
            row += 1
    assert row == want_count
    # start positions of zero: the relative rule
    _, f0, s_zero = O.prefill(q, k, v, g, beta, cu, initial_state=S0,
                              snapshot_interval=interval, start_pos=[0] * len(lens))
    _, f1, s_none = O.prefill(q, k, v, g, beta, cu, initial_state=S0,
                              snapshot_interval=interval)
    assert np.array_equal(s_zero, s_none) and np.array_equal(f0, f1)
    assert s_none.shape[0] == sum(L // interval for L in lens)


ALL_PINS = [pin_exact_write, pin_beta_zero, pin_split_resume, pin_product_form,
            pin_exact_rational, pin_orthonormal_recall, pin_scalar_iir,
            pin_linearity, pin_contraction, pin_permutation, pin_frozen_state,
            pin_varlen_packing, pin_decode_matches_prefill, pin_absolute_snapshots]
