"""fp64 model of the chunked prefill decomposition, with optional emulation of
the HIP kernels' operand roundings.

TEST INFRASTRUCTURE (CPU only).  This is neither the oracle nor the product:
it restates, in numpy, the algebra the prefill kernels evaluate, so that

* the decomposition itself is pinned to the token-by-token oracle on the CPU
  (in exact fp64 arithmetic the two agree to ~1e-12), and
* the effect of each rounding point of the kernels (which operand is a bf16,
  a bf16 hi + lo pair, or an fp16 value with a power-of-two exponent per
  tile) can be measured against the oracle without a GPU.

It shares no code with the HIP path or with the oracle.

The chunked form ("Kimi K3 technical FAQ", question "What is KDA, and why
does a serving engineer care?": the state is updated per chunk, parallel
within a chunk and recurrent across chunks).  With C-row chunks restarting at
every sequence start, G the inclusive cumulative sum of g inside the chunk,
G_C its last row and S the state at the chunk start:

    A_ts = b_t sum_c k_t[c] k_s[c] e^{G_t[c] - G_s[c]}   (s < t)
    B_ts =     sum_c q_t[c] k_s[c] e^{G_t[c] - G_s[c]}   (s <= t)
    T = (I + A)^-1,  TB = T Diag(b),  Kt = K . e^G,  W = TB Kt,  M = B TB
    Q' = Q . e^G - M Kt,  U~ = TB V,  O~ = M V,  Kd = (K . e^{G_C - G})^T
    U = U~ - W S,  O = scale (Q' S + O~),  S' = Diag(e^{G_C}) S + Kd U

Substituting the recurrence S_t = (I - b_t k_t k_t^T) Diag(e^{g_t}) S_{t-1} +
b_t k_t v_t^T into itself inside a chunk gives (I + A) U = Diag(b)(V - Kt S)
for the per-token write vectors U, hence the lines above.

The Gram matrices are formed blockwise (16 x 16 blocks) around a reference
row, as the kernel forms them on the matrix unit: a diagonal block (R, R)
factorises e^{G_t - G_s} = e^{G_t - r} e^{r - G_s} with r = G at row
16R + 7, an off-diagonal block (R, s < R) with r = G at row 16R - 1.  In
exact arithmetic the factorisation changes nothing.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Callable, Dict, Optional

import numpy as np

C = 64
BLK = 16


# ---------------------------------------------------------------------------
# rounding helpers (fp64 in, fp64 out)
# ---------------------------------------------------------------------------
def to_f32(x):
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def to_bf16(x):
    """Round to bf16 (nearest even) through fp32."""
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return r.astype(np.uint32).view(np.float32).astype(np.float64)


def to_f16(x):
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float16).astype(np.float64)


def bf16_hilo(x):
    """x (fp32) as hi + lo, both bf16: the kernels' three-pass operands keep
    hi*hi + hi*lo + lo*hi of a product."""
    x = to_f32(x)
    hi = to_bf16(x)
    lo = to_bf16(x - hi)
    return hi, lo


def hilo_product(a, b):
    """a @ b with both operands split into bf16 hi + lo, three passes."""
    ah, al = bf16_hilo(a)
    bh, bl = bf16_hilo(b)
    return ah @ bh + ah @ bl + al @ bh


def frexp_bound(m):
    """e with m < 2^e (frexp's exponent); -126 for zero."""
    if m == 0.0 or not np.isfinite(m):
        return -126
    return int(np.frexp(m)[1])


def f16_scaled(x, top=15):
    """One fp16 rounding of a whole tile stored times 2^(top - e), e the
    bound exponent of its largest magnitude, then scaled back."""
    x = to_f32(x)
    e = frexp_bound(float(np.max(np.abs(x))) if x.size else 0.0)
    s = float(2.0 ** (top - e))
    return to_f16(x * s) / s


def f16_hilo_scaled(x, top=15):
    x = to_f32(x)
    e = frexp_bound(float(np.max(np.abs(x))) if x.size else 0.0)
    s = float(2.0 ** (top - e))
    y = x * s
    hi = to_f16(y)
    lo = to_f16(y - hi)
    return (hi + lo) / s


# token row of row r in token tile mt (the kernels' renumbering inside a chunk)
def tok_of(mt, r):
    return ((mt >> 1) << 5) + ((r >> 2) << 3) + ((mt & 1) << 2) + (r & 3)


# state row (within a 32-row block) of row r in row tile m
def chan_of(m, r):
    return ((r >> 2) << 3) + (m << 2) + (r & 3)


TOKEN_TILES = [np.array([tok_of(mt, r) for r in range(16)]) for mt in range(4)]
CHAN_TILES = [np.array([chan_of(m, r) for r in range(16)]) for m in range(2)]


def per_tile_w(Wm, fn):
    """W or Q' [C, dk]: tiles of 16 tokens (a token tile) x 32 channels."""
    out = np.array(Wm, dtype=np.float64)
    dk = Wm.shape[1]
    for mt in range(4):
        rows = TOKEN_TILES[mt]
        for r in range(0, dk, 32):
            out[np.ix_(rows, np.arange(r, min(r + 32, dk)))] = fn(
                Wm[np.ix_(rows, np.arange(r, min(r + 32, dk)))])
    return out


def per_tile_kd(Kd, fn):
    """Kd [dk, C]: tiles of 16 channels (row tile m of a 32-row block) x 32 tokens."""
    out = np.array(Kd, dtype=np.float64)
    dk = Kd.shape[0]
    for w in range(0, dk, 32):
        for m in range(2):
            rows = w + CHAN_TILES[m]
            rows = rows[rows < dk]
            for ks in range(2):
                cols = np.arange(32 * ks, 32 * ks + 32)
                if rows.size:
                    out[np.ix_(rows, cols)] = fn(Kd[np.ix_(rows, cols)])
    return out


# ---------------------------------------------------------------------------
# rounding plans
# ---------------------------------------------------------------------------
@dataclass
class Rounding:
    """Where the kernels round.  Every field None = exact fp64 arithmetic."""
    gram_diag_A: Optional[Callable] = None   # (X, Y) -> X @ Y.T for diagonal A blocks
    gram_diag_B: Optional[Callable] = None
    gram_off: Optional[Callable] = None      # off-diagonal A and B blocks
    solve: Optional[Callable] = None         # (TB, B) -> M = B TB
    ktilde: Optional[Callable] = None        # K e^G as used in W and Q'
    w_prod: Optional[Callable] = None        # (TB, Kt) -> TB Kt
    v_prod: Optional[Callable] = None        # (TB or M, V) -> product
    scan_w: Optional[Callable] = None        # W, Q' operand tiles of the scan
    scan_kd: Optional[Callable] = None
    scan_state: Optional[Callable] = None    # S operand (per 32-row block, per value tile)
    scan_u: Optional[Callable] = None        # U operand
    extra: Dict[str, object] = field(default_factory=dict)


EXACT = Rounding()


def _mm(fn, a, b):
    return a @ b if fn is None else fn(a, b)


def kernel_rounding(ktilde="hilo", diag_a="hilo", scan_ops="f16") -> Rounding:
    """The rounding points of the HIP kernels (the defaults are the kernels'
    current choices; the alternatives are the earlier ones, kept so that the
    reason for each choice stays measurable).

    ktilde:   "hilo" (K e^G as a bf16 hi + lo pair in W = TB Kt and M Kt),
              "bf16" (one bf16 rounding).
    diag_a:   "hilo" (diagonal A blocks in three passes, as B's), "bf16" (one
              bf16 rounding of the row factor times the bf16 hi of the column
              factor).
    scan_ops: "f16" (W, Q', Kd as fp16 with one power-of-two exponent per
              16 x 32 tile), "bf16" (one bf16 rounding each).
    """
    def gram_diag_A(X, Y):
        if diag_a == "bf16":
            return to_bf16(X) @ to_bf16(Y).T
        return hilo_product(X, Y.T)

    def gram_diag_B(X, Y):
        return hilo_product(X, Y.T)

    def gram_off(X, Y):
        return to_f16(X) @ to_f16(Y).T

    def kt(x):
        if ktilde == "bf16":
            return to_bf16(x)
        return x  # the hi + lo pair is carried into the product (w_prod)

    def w_prod(TB, Kt):
        if ktilde == "bf16":
            th, tl = bf16_hilo(TB)
            return th @ Kt + tl @ Kt
        return hilo_product(TB, Kt)

    def v_prod(Tm, V):
        th, tl = bf16_hilo(Tm)
        vh, vl = bf16_hilo(V)
        return th @ vh + tl @ vh + th @ vl

    def scan_state(S):
        return f16_hilo_scaled(S)

    def scan_u(U):
        return f16_hilo_scaled(U)

    if scan_ops == "f16":
        sw = lambda x: per_tile_w(x, f16_scaled)
        sk = lambda x: per_tile_kd(x, f16_scaled)
    else:
        sw = sk = to_bf16
    return Rounding(gram_diag_A=gram_diag_A, gram_diag_B=gram_diag_B, gram_off=gram_off,
                    solve=lambda TB, B: hilo_product(B, TB), ktilde=kt, w_prod=w_prod,
                    v_prod=v_prod, scan_w=sw, scan_kd=sk, scan_state=scan_state,
                    scan_u=scan_u)


# ---------------------------------------------------------------------------
# prep: the state-independent quantities of one chunk
# ---------------------------------------------------------------------------
@dataclass
class ChunkOps:
    W: np.ndarray     # [C, dk]
    Qp: np.ndarray    # [C, dk]
    Kd: np.ndarray    # [dk, C]
    Ut: np.ndarray    # [C, dv]
    Ot: np.ndarray    # [C, dv]
    dec: np.ndarray   # [dk]


def gram(q, k, G, beta, rnd: Rounding):
    """A (strictly lower, times beta_t) and B (lower incl. diagonal), blockwise."""
    n = q.shape[0]
    A = np.zeros((n, n))
    B = np.zeros((n, n))
    for R in range(n // BLK):
        t = slice(BLK * R, BLK * R + BLK)
        # diagonal block
        r = G[BLK * R + 7]
        X = k[t] * np.exp(G[t] - r)
        Xq = q[t] * np.exp(G[t] - r)
        Y = k[t] * np.exp(r - G[t])
        A[t, t] = X @ Y.T if rnd.gram_diag_A is None else rnd.gram_diag_A(X, Y)
        B[t, t] = Xq @ Y.T if rnd.gram_diag_B is None else rnd.gram_diag_B(Xq, Y)
        # off-diagonal blocks
        if R > 0:
            r = G[BLK * R - 1]
            X = k[t] * np.exp(G[t] - r)
            Xq = q[t] * np.exp(G[t] - r)
            for ts in range(R):
                s = slice(BLK * ts, BLK * ts + BLK)
                Y = k[s] * np.exp(r - G[s])
                if rnd.gram_off is None:
                    A[t, s] = X @ Y.T
                    B[t, s] = Xq @ Y.T
                else:
                    A[t, s] = rnd.gram_off(X, Y)
                    B[t, s] = rnd.gram_off(Xq, Y)
    A = np.tril(A, -1) * beta[:, None]
    B = np.tril(B)
    return A, B


def prep_chunk(q, k, v, g, beta, rnd: Rounding = EXACT) -> ChunkOps:
    """One chunk, rows zero-padded to C (padding rows: q = k = v = 0, g = 0,
    beta = 0, which leave the state alone)."""
    G = np.cumsum(g, axis=0)
    A, B = gram(q, k, G, beta, rnd)
    n = q.shape[0]
    T = np.linalg.solve(np.eye(n) + A, np.eye(n))  # unit lower-triangular system
    TB = T * beta[None, :]
    eG = np.exp(G)
    Kt = k * eG
    Ktr = Kt if rnd.ktilde is None else rnd.ktilde(Kt)
    W = _mm(rnd.w_prod, TB, Ktr)
    M = B @ TB if rnd.solve is None else rnd.solve(TB, B)
    Qp = q * eG - _mm(rnd.w_prod, M, Ktr)
    Ut = _mm(rnd.v_prod, TB, v)
    Ot = _mm(rnd.v_prod, M, v)
    Kd = (k * np.exp(G[-1][None, :] - G)).T
    if rnd.scan_w is not None:
        W = rnd.scan_w(W)
        Qp = rnd.scan_w(Qp)
    if rnd.scan_kd is not None:
        Kd = rnd.scan_kd(Kd)
    return ChunkOps(W, Qp, Kd, Ut, Ot, np.exp(G[-1]))


# ---------------------------------------------------------------------------
# scan: the recurrence over chunks
# ---------------------------------------------------------------------------
def scan_chunk(S, ops: ChunkOps, scale: float, rnd: Rounding = EXACT):
    """Returns (O [C, dv], S')."""
    Sop = S
    if rnd.scan_state is not None:
        # one exponent per 32-row block and 16-column value tile
        Sop = np.array(S)
        for r in range(0, S.shape[0], 32):
            for j in range(0, S.shape[1], 16):
                Sop[r:r + 32, j:j + 16] = rnd.scan_state(S[r:r + 32, j:j + 16])
    U = ops.Ut - ops.W @ Sop
    O = scale * (ops.Qp @ Sop + ops.Ot)
    Uop = U
    if rnd.scan_u is not None:
        Uop = np.array(U)
        for t in range(0, U.shape[0], 32):
            for j in range(0, U.shape[1], 16):
                Uop[t:t + 32, j:j + 16] = rnd.scan_u(U[t:t + 32, j:j + 16])
    Sn = ops.dec[:, None] * S + ops.Kd @ Uop
    return O, Sn


def prefill(q, k, v, g, beta, cu_seqlens, initial_state=None, snapshot_interval=0,
            scale=None, rnd: Rounding = EXACT):
    """Chunked prefill of packed sequences [T, H, d] (numpy, any float dtype;
    values are taken as given).  Returns (out [T, H, dv], final [N, H, dk, dv],
    snapshots [count, H, dk, dv]) like the oracle."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    beta = np.asarray(beta, dtype=np.float64)
    cu = [int(x) for x in np.asarray(cu_seqlens)]
    T, H, dk = q.shape
    dv = v.shape[2]
    N = len(cu) - 1
    sc = 1.0 / np.sqrt(dk) if scale is None else float(scale)
    out = np.zeros((T, H, dv))
    final = np.zeros((N, H, dk, dv))
    snaps = []
    for b in range(N):
        s0, e0 = cu[b], cu[b + 1]
        L = e0 - s0
        seq_snaps = [np.zeros((H, dk, dv)) for _ in range(L // snapshot_interval)] \
            if snapshot_interval else []
        for h in range(H):
            S = np.zeros((dk, dv)) if initial_state is None else \
                np.array(initial_state[b, h], dtype=np.float64)
            for c0 in range(0, L, C):
                n = min(C, L - c0)
                rows = slice(s0 + c0, s0 + c0 + n)

                def pad(x):
                    z = np.zeros((C,) + x.shape[1:])
                    z[:n] = x
                    return z
                ops = prep_chunk(pad(q[rows, h]), pad(k[rows, h]), pad(v[rows, h]),
                                 pad(g[rows, h]), pad(beta[rows, h]), rnd)
                O, S = scan_chunk(S, ops, sc, rnd)
                out[rows, h] = O[:n]
                if snapshot_interval and (c0 + n) % snapshot_interval == 0:
                    seq_snaps[(c0 + n) // snapshot_interval - 1][h] = S
            final[b, h] = S
        snaps.extend(seq_snaps)
    snaps = np.stack(snaps) if snaps else np.zeros((0, H, dk, dv))
    return out, final, snaps
