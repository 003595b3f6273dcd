"""fp64 token-by-token CPU oracle for the Kimi Delta Attention recurrence.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` import this package.  It shares no code with
the HIP path and never imports it.

The arithmetic lives in ``kda_oracle.c`` (plain C, fp64); this module only
compiles it with gcc and marshals numpy arrays through ctypes.  What is
computed, and the passages it follows, are stated in the header of
``kda_oracle.c``:

* "Kimi K3 technical FAQ", question "What is KDA, and why does a serving
  engineer care?": delta-rule recurrence with a per-channel forget gate and a
  dk x dv state per head, read as
  ``S_t = (I - b_t k_t k_t^T) Diag(a_t) S_{t-1} + b_t k_t v_t^T``,
  ``o_t = dk^-1/2 S_t^T q_t``.
* "Day-0 vLLM support for Kimi K3", section "Kimi K3's architecture, and how
  vLLM serves it": state snapshots at block boundaries for prefix reuse.
* "Kimi K3 technical FAQ", same question: queries and keys pass through a
  short convolution, Swish and L2 normalisation first (``qk_frontend``).
* "Kimi K3 technical FAQ", question "What does the architecture actually
  look like?", and the vLLM page's architecture section: Attention Residuals,
  a softmax over earlier block outputs with a learned pseudo-query, residual
  add and RMSNorm (``attnres``).

Parity pins for every function here are in ``tests/test_oracle_pins.py``
and ``tests/test_frontend_pins.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "kda_oracle.c")
LIBRARY = os.path.join(_HERE, "libkda_oracle.so")


def build(src: str = SOURCE, out: str = LIBRARY) -> str:
    """Compile the oracle with gcc (-O2, no fast-math, no SIMD intrinsics)."""
    tmp = out + ".tmp"
    cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-pthread",
           "-fno-fast-math", "-o", tmp, src, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def _bind(lib: ctypes.CDLL) -> ctypes.CDLL:
    P = ctypes.c_void_p
    i32, i64, f64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_double
    lib.kda_oracle_prefill.restype = ctypes.c_int
    lib.kda_oracle_prefill.argtypes = [i32, P, P, i32, i32, i32, P, P, P, P, P,
                                       P, f64, i64, P, P, P, i32]
    lib.kda_oracle_decode.restype = ctypes.c_int
    lib.kda_oracle_decode.argtypes = [i32, i32, i32, i32, i32, P, P, P, P, P,
                                      P, P, f64, P, i32]
    lib.kda_oracle_snapshot_count.restype = i64
    lib.kda_oracle_snapshot_count.argtypes = [i32, P, P, i64]
    lib.kda_oracle_attnres.restype = ctypes.c_int
    lib.kda_oracle_attnres.argtypes = [i32, i64, i32, P, P, P, P, f64, f64, P, P]
    lib.kda_oracle_qk_frontend.restype = ctypes.c_int
    lib.kda_oracle_qk_frontend.argtypes = [i32, P, i32, i32, i32, P, P, P, P, f64, P, P]
    return lib


class Oracle:
    """ctypes handle on one compiled oracle library (the real one, or a
    deliberately mutated copy built by the mutation tests)."""

    def __init__(self, path: str = LIBRARY):
        if not os.path.exists(path):
            if path != LIBRARY:
                raise FileNotFoundError(path)
            build()
        self.path = path
        self.lib = _bind(ctypes.CDLL(path))

    @staticmethod
    def _threads(nthreads: Optional[int]) -> int:
        if nthreads:
            return int(nthreads)
        try:
            return max(1, len(os.sched_getaffinity(0)))
        except AttributeError:  # pragma: no cover
            return max(1, os.cpu_count() or 1)

    @staticmethod
    def _f32(x) -> np.ndarray:
        return np.ascontiguousarray(np.asarray(x, dtype=np.float32))

    @staticmethod
    def _starts(start_pos, n):
        if start_pos is None:
            return None
        st = np.ascontiguousarray(np.asarray(start_pos, dtype=np.int64))
        assert st.shape == (n,)
        return st

    def snapshot_count(self, cu_seqlens, interval: int, start_pos=None) -> int:
        cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64))
        st = self._starts(start_pos, len(cu) - 1)
        return int(self.lib.kda_oracle_snapshot_count(
            len(cu) - 1, cu.ctypes.data, None if st is None else st.ctypes.data, int(interval)))

    def prefill(self, q, k, v, g, beta, cu_seqlens, initial_state=None,
                scale: float = 0.0, snapshot_interval: int = 0,
                nthreads: Optional[int] = None, start_pos=None):
        """Run every (sequence, head) token by token in fp64.

        start_pos: [N] absolute position of each sequence's first token
        (default 0): snapshots are taken at the absolute multiples of the
        interval.

        q, k, g: [T, H, dk]; v: [T, H, dv]; beta: [T, H] (any float dtype,
        converted exactly to fp32).  initial_state: [N, H, dk, dv] or None,
        converted to fp64.  Returns (out [T,H,dv], final [N,H,dk,dv],
        snapshots [count,H,dk,dv]) as fp64 arrays.
        """
        q, k, v, g, beta = (self._f32(a) for a in (q, k, v, g, beta))
        T, H, dk = q.shape
        dv = v.shape[2]
        assert k.shape == (T, H, dk) and g.shape == (T, H, dk)
        assert v.shape == (T, H, dv) and beta.shape == (T, H)
        cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64))
        N = len(cu) - 1
        assert cu[0] == 0 and cu[-1] == T
        init = None
        if initial_state is not None:
            init = np.ascontiguousarray(np.asarray(initial_state, dtype=np.float64))
            assert init.shape == (N, H, dk, dv)
        out = np.zeros((T, H, dv), dtype=np.float64)
        final = np.zeros((N, H, dk, dv), dtype=np.float64)
        st = self._starts(start_pos, N)
        count = self.snapshot_count(cu, snapshot_interval, start_pos=st)
        snaps = np.zeros((count, H, dk, dv), dtype=np.float64)
        rc = self.lib.kda_oracle_prefill(
            N, cu.ctypes.data, None if st is None else st.ctypes.data, H, dk, dv,
            q.ctypes.data, k.ctypes.data,
            v.ctypes.data, g.ctypes.data, beta.ctypes.data,
            None if init is None else init.ctypes.data, float(scale),
            int(snapshot_interval), out.ctypes.data, final.ctypes.data,
            snaps.ctypes.data if count else None, self._threads(nthreads))
        if rc != 0:
            raise ValueError("kda_oracle_prefill rejected its arguments")
        return out, final, snaps

    def decode(self, q, k, v, g, beta, state, slots=None, scale: float = 0.0,
               nthreads: Optional[int] = None):
        """``steps`` chained single-token steps.

        q, k, g: [steps, N, H, dk]; v: [steps, N, H, dv]; beta: [steps, N, H];
        state: [S, H, dk, dv] (copied to fp64; the updated copy is returned).
        Returns (out [steps, N, H, dv], state).
        """
        q, k, v, g, beta = (self._f32(a) for a in (q, k, v, g, beta))
        steps, N, H, dk = q.shape
        dv = v.shape[3]
        st = np.array(state, dtype=np.float64, order="C", copy=True)
        sl = None
        if slots is not None:
            sl = np.ascontiguousarray(np.asarray(slots, dtype=np.int32))
            assert sl.shape == (N,)
        out = np.zeros((steps, N, H, dv), dtype=np.float64)
        rc = self.lib.kda_oracle_decode(
            steps, N, H, dk, dv, q.ctypes.data, k.ctypes.data, v.ctypes.data,
            g.ctypes.data, beta.ctypes.data, st.ctypes.data,
            None if sl is None else sl.ctypes.data, float(scale),
            out.ctypes.data, self._threads(nthreads))
        if rc != 0:
            raise ValueError("kda_oracle_decode rejected its arguments")
        return out, st


    def qk_frontend(self, x, w, cu_seqlens, conv_width: int, eps: float,
                    state=None, slots=None, num_slots: Optional[int] = None):
        """Short convolution -> Swish -> L2 norm of one tensor (q or k).

        x: [T, H, dk]; w: [H*dk, W] (or [H, dk, W]) convolution taps, tap W-1
        on the current token; state: [S, W-1, H, dk] inputs that preceded each
        slot's sequence (oldest first) or None for zero history; slots: [N]
        state row of each sequence or None (identity).  Returns (y [T,H,dk]
        fp64, new_state [S, W-1, H, dk] fp32): a copy of ``state`` (zeros when
        it is None) whose rows of this call's sequences hold their last W-1
        inputs.
        """
        x = self._f32(x)
        T, H, dk = x.shape
        W = int(conv_width)
        w = self._f32(w).reshape(H * dk, W)
        cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64))
        N = len(cu) - 1
        assert cu[0] == 0 and cu[-1] == T
        sl = None
        if slots is not None:
            sl = np.ascontiguousarray(np.asarray(slots, dtype=np.int32))
            assert sl.shape == (N,)
        if state is not None:
            new_state = np.array(state, dtype=np.float32, order="C", copy=True)
            S = new_state.shape[0]
            assert new_state.shape == (S, W - 1, H, dk)
            st_in = new_state.copy()
        else:
            S = num_slots if num_slots is not None else (
                N if sl is None else int(sl.max(initial=-1)) + 1)
            new_state = np.zeros((S, W - 1, H, dk), dtype=np.float32)
            st_in = None
        if sl is not None and N:
            assert sl.min() >= 0 and sl.max() < S and len(set(sl.tolist())) == N
        else:
            assert N <= S
        y = np.zeros((T, H, dk), dtype=np.float64)
        rc = self.lib.kda_oracle_qk_frontend(
            N, cu.ctypes.data, H, dk, W, x.ctypes.data, w.ctypes.data,
            None if st_in is None else st_in.ctypes.data,
            None if sl is None else sl.ctypes.data, float(eps), y.ctypes.data,
            new_state.ctypes.data)
        if rc != 0:
            raise ValueError("kda_oracle_qk_frontend rejected its arguments")
        return y, new_state


    def attnres(self, sources, w, x=None, gamma=None, scale: float = 1.0, eps: float = 1e-6):
        """Attention Residuals aggregation of one layer's input.

        sources: [M, T, d] (or a list of M [T, d] arrays); w, gamma: [d];
        x: [T, d] residual or None.  Returns (h, y) [T, d] fp64.
        """
        src = np.ascontiguousarray(np.stack([self._f32(s) for s in sources]))
        M, T, d = src.shape
        wv = self._f32(w).reshape(d)
        xv = None if x is None else self._f32(x).reshape(T, d)
        gv = None if gamma is None else self._f32(gamma).reshape(d)
        h = np.zeros((T, d), dtype=np.float64)
        y = np.zeros((T, d), dtype=np.float64)
        rc = self.lib.kda_oracle_attnres(
            M, T, d, src.ctypes.data, None if xv is None else xv.ctypes.data, wv.ctypes.data,
            None if gv is None else gv.ctypes.data, float(scale), float(eps), h.ctypes.data,
            y.ctypes.data)
        if rc != 0:
            raise ValueError("kda_oracle_attnres rejected its arguments")
        return h, y


_DEFAULT: Optional[Oracle] = None


def get() -> Oracle:
    """The oracle built from ``kda_oracle.c`` (compiled on first use)."""
    global _DEFAULT
    if _DEFAULT is None:
        _DEFAULT = Oracle()
    return _DEFAULT


def prefill(*args, **kwargs):
    return get().prefill(*args, **kwargs)


def decode(*args, **kwargs):
    return get().decode(*args, **kwargs)


def qk_frontend(*args, **kwargs):
    return get().qk_frontend(*args, **kwargs)


def attnres(*args, **kwargs):
    return get().attnres(*args, **kwargs)
