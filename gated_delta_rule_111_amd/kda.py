"""Thin Python binding of libkda (include/kda.h).

Argument marshalling only: this module checks dtypes, shapes, devices and
contiguity of torch tensors, allocates outputs with torch when the caller
does not pass them, and hands raw device pointers plus the current HIP stream
to the C ABI.  Every step of the computation runs in the HIP kernels.  If the
shared library has not been built the first call raises; there is no other
path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence, Tuple

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIBRARY = os.path.join(_PKG, "libkda.so")

KDA_BF16, KDA_F32 = 0, 1
_STATUS = {0: "KDA_OK", 1: "KDA_ERR_INVALID_ARG", 2: "KDA_ERR_UNSUPPORTED",
           3: "KDA_ERR_ALIGNMENT", 4: "KDA_ERR_WORKSPACE", 5: "KDA_ERR_HIP"}


class KdaError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{_STATUS.get(status, status)}: {detail}")
        self.status = status
        self.detail = detail


class Config(ctypes.Structure):
    _fields_ = [("num_heads", ctypes.c_int32), ("dk", ctypes.c_int32),
                ("dv", ctypes.c_int32), ("in_dtype", ctypes.c_int),
                ("out_dtype", ctypes.c_int), ("scale", ctypes.c_float)]


class FrontendConfig(ctypes.Structure):
    _fields_ = [("num_heads", ctypes.c_int32), ("dk", ctypes.c_int32),
                ("conv_width", ctypes.c_int32), ("in_dtype", ctypes.c_int),
                ("out_dtype", ctypes.c_int), ("eps", ctypes.c_float)]


_lib: Optional[ctypes.CDLL] = None


def load(path: str = LIBRARY) -> ctypes.CDLL:
    """Load libkda.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with `python -m gated_delta_rule_111_amd.build` "
            "(libkda has no fallback path)")
    lib = ctypes.CDLL(path)
    P, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    CP = ctypes.POINTER(Config)
    lib.kda_version.restype = i32
    lib.kda_status_string.restype = ctypes.c_char_p
    lib.kda_status_string.argtypes = [ctypes.c_int]
    lib.kda_last_error_detail.restype = ctypes.c_char_p
    lib.kda_snapshot_count.restype = i64
    lib.kda_snapshot_count.argtypes = [P, i32, i32]
    lib.kda_prefill_workspace_size.restype = sz
    lib.kda_prefill_workspace_size.argtypes = [CP, i32, i64]
    lib.kda_prefill.restype = ctypes.c_int
    lib.kda_prefill.argtypes = [CP, i32, P, P, P, P, P, P, P, P, P, P, i32, P, P, sz, P]
    lib.kda_prefill_noalloc.restype = ctypes.c_int
    lib.kda_prefill_noalloc.argtypes = [CP, i32, P, P, P, P, P, P, P, P, P, P, i32, P, P]
    lib.kda_decode.restype = ctypes.c_int
    lib.kda_decode.argtypes = [CP, i32, P, P, P, P, P, P, P, P, P]
    lib.kda_attnres.restype = ctypes.c_int
    lib.kda_attnres.argtypes = [ctypes.c_void_p, i64, P, P, P, P, P, P, P]
    lib.kda_prefill_pool.restype = ctypes.c_int
    lib.kda_prefill_pool.argtypes = [CP, i32, P, P, P, P, P, P, P, P, P, P, P, i32, P, i32, P, P,
                                     sz, P]
    lib.kda_snapshot_count_at.restype = i64
    lib.kda_snapshot_count_at.argtypes = [P, P, i32, i32]
    lib.kda_prefill_pool_workspace_size.restype = sz
    lib.kda_prefill_pool_workspace_size.argtypes = [CP, i32, i64]
    lib.kda_decode_spec_step.restype = ctypes.c_int
    lib.kda_decode_spec_step.argtypes = [CP, i32, i32, P, P, P, P, P, P, P, P, P, P, P, P, P,
                                         P]
    lib.kda_decode_multi.restype = ctypes.c_int
    lib.kda_decode_multi.argtypes = [CP, i32, i32, ctypes.c_int, P, P, P, P, P, P, P, P, P, P]
    lib.kda_qk_frontend.restype = ctypes.c_int
    lib.kda_qk_frontend.argtypes = [ctypes.POINTER(FrontendConfig), i32, P, P, P, P, P, P,
                                    P, P, P, P, P, i32, P, P, P]
    _lib = lib
    return lib


def _dtype_code(dt: torch.dtype) -> int:
    if dt == torch.bfloat16:
        return KDA_BF16
    if dt == torch.float32:
        return KDA_F32
    raise TypeError(f"unsupported dtype {dt}; use torch.bfloat16 or torch.float32")


def _check(status: int):
    if status != 0:
        raise KdaError(status, load().kda_last_error_detail().decode())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _need(t: torch.Tensor, name: str, shape, dtype, device):
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)} != {tuple(shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name}: dtype {t.dtype} != {dtype}")
    if t.device != device:
        raise ValueError(f"{name}: on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")


def _stream(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _empty(stream, *shape, dtype, device) -> torch.Tensor:
    """torch.empty from the pool of the stream the kernels run on.  The
    caching allocator orders a block's reuse only on the stream it was
    allocated on: a workspace taken from the current stream's pool and
    freed on return could be handed to the next allocation there while the
    kernels enqueued on ``stream`` still read it."""
    if stream is None:
        return torch.empty(*shape, dtype=dtype, device=device)
    with torch.cuda.stream(stream):
        return torch.empty(*shape, dtype=dtype, device=device)


def config(H: int, dk: int, dv: int, in_dtype: torch.dtype,
           out_dtype: torch.dtype = torch.float32, scale: float = 0.0) -> Config:
    return Config(H, dk, dv, _dtype_code(in_dtype), _dtype_code(out_dtype), float(scale))


def snapshot_count(cu_seqlens_host: Sequence[int], interval: int) -> int:
    cu = (ctypes.c_int32 * len(cu_seqlens_host))(*cu_seqlens_host)
    n = load().kda_snapshot_count(cu, len(cu_seqlens_host) - 1, int(interval))
    if n < 0:
        raise ValueError("cu_seqlens must be non-decreasing")
    return int(n)


def workspace_size(cfg: Config, num_seqs: int, total_tokens: int) -> int:
    return int(load().kda_prefill_workspace_size(ctypes.byref(cfg), num_seqs, total_tokens))


def prefill(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
            beta: torch.Tensor, cu_seqlens: torch.Tensor,
            initial_state: Optional[torch.Tensor] = None, snapshot_interval: int = 0,
            out_dtype: Optional[torch.dtype] = None, scale: float = 0.0,
            cu_seqlens_host: Optional[Sequence[int]] = None,
            out: Optional[torch.Tensor] = None, final_state: Optional[torch.Tensor] = None,
            snapshots: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
            stream=None) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """kda_prefill on packed varlen sequences; returns (out, final_state, snapshots).

    q, k: [T, H, dk]; v: [T, H, dv] (bf16 or fp32, same dtype); g: [T, H, dk]
    fp32 log-gates; beta: [T, H] fp32; cu_seqlens: [N+1] int32 on the device
    (cu_seqlens_host, if given, must hold the same offsets and avoids a copy).
    """
    lib = load()
    dev = q.device
    T, H, dk = q.shape
    dv = v.shape[2]
    if cu_seqlens_host is None:
        cu_seqlens_host = cu_seqlens.cpu().tolist()
    cu_list = [int(x) for x in cu_seqlens_host]
    N = len(cu_list) - 1
    _need(cu_seqlens, "cu_seqlens", (N + 1,), torch.int32, dev)
    for name, t, shp, dt in (("q", q, (T, H, dk), q.dtype), ("k", k, (T, H, dk), q.dtype),
                             ("v", v, (T, H, dv), q.dtype), ("g", g, (T, H, dk), torch.float32),
                             ("beta", beta, (T, H), torch.float32)):
        _need(t, name, shp, dt, dev)
    if cu_list[-1] != T:
        raise ValueError(f"cu_seqlens ends at {cu_list[-1]} but q has {T} tokens")
    if initial_state is not None:
        _need(initial_state, "initial_state", (N, H, dk, dv), torch.float32, dev)
    if out_dtype is None:
        out_dtype = out.dtype if out is not None else torch.float32
    cfg = config(H, dk, dv, q.dtype, out_dtype, scale)
    nsnap = snapshot_count(cu_list, snapshot_interval) if snapshot_interval > 0 else 0
    if out is None:
        out = _empty(stream, T, H, dv, dtype=out_dtype, device=dev)
    _need(out, "out", (T, H, dv), out_dtype, dev)
    if final_state is None:
        final_state = _empty(stream, N, H, dk, dv, dtype=torch.float32, device=dev)
    _need(final_state, "final_state", (N, H, dk, dv), torch.float32, dev)
    if snapshots is None:
        snapshots = _empty(stream, nsnap, H, dk, dv, dtype=torch.float32, device=dev)
    _need(snapshots, "snapshots", (nsnap, H, dk, dv), torch.float32, dev)
    ws_bytes = workspace_size(cfg, N, T)
    if workspace is None and ws_bytes > 0:
        workspace = _empty(stream, ws_bytes, dtype=torch.uint8, device=dev)
    cu_arr = (ctypes.c_int32 * len(cu_list))(*cu_list)
    _check(lib.kda_prefill(
        ctypes.byref(cfg), N, cu_arr, cu_seqlens.data_ptr(), q.data_ptr(), k.data_ptr(),
        v.data_ptr(), g.data_ptr(), beta.data_ptr(), _ptr(initial_state), out.data_ptr(),
        final_state.data_ptr(), int(snapshot_interval),
        snapshots.data_ptr() if nsnap > 0 else None, _ptr(workspace),
        workspace.numel() if workspace is not None else 0, _stream(stream)))
    return out, final_state, snapshots


NOALLOC_SCRATCH_BYTES = 128 * 1024 * 1024  # KDA_NOALLOC_SCRATCH_BYTES


def prefill_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
                    beta: torch.Tensor, cu_seqlens: torch.Tensor,
                    initial_state: Optional[torch.Tensor] = None, snapshot_interval: int = 0,
                    cu_seqlens_host: Optional[Sequence[int]] = None,
                    out: Optional[torch.Tensor] = None,
                    final_state: Optional[torch.Tensor] = None,
                    snapshots: Optional[torch.Tensor] = None, scale: float = 0.0,
                    stream=None) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """kda_prefill_noalloc: kda_prefill with the chunk operands in the
    library's fixed per-GPU array (no workspace).  Pass out, final_state and
    snapshots (and cu_seqlens_host) to make the call allocate nothing on the
    Python side either; whatever is not passed is allocated here."""
    lib = load()
    dev = q.device
    T, H, dk = q.shape
    dv = v.shape[2]
    if cu_seqlens_host is None:
        cu_seqlens_host = cu_seqlens.cpu().tolist()
    cu_list = [int(x) for x in cu_seqlens_host]
    N = len(cu_list) - 1
    _need(cu_seqlens, "cu_seqlens", (N + 1,), torch.int32, dev)
    for name, t, shp, dt in (("q", q, (T, H, dk), q.dtype), ("k", k, (T, H, dk), q.dtype),
                             ("v", v, (T, H, dv), q.dtype), ("g", g, (T, H, dk), torch.float32),
                             ("beta", beta, (T, H), torch.float32)):
        _need(t, name, shp, dt, dev)
    if cu_list[-1] != T:
        raise ValueError(f"cu_seqlens ends at {cu_list[-1]} but q has {T} tokens")
    if initial_state is not None:
        _need(initial_state, "initial_state", (N, H, dk, dv), torch.float32, dev)
    out_dtype = out.dtype if out is not None else torch.float32
    cfg = config(H, dk, dv, q.dtype, out_dtype, scale)
    nsnap = snapshot_count(cu_list, snapshot_interval) if snapshot_interval > 0 else 0
    if out is None:
        out = _empty(stream, T, H, dv, dtype=out_dtype, device=dev)
    _need(out, "out", (T, H, dv), out_dtype, dev)
    if final_state is None:
        final_state = _empty(stream, N, H, dk, dv, dtype=torch.float32, device=dev)
    _need(final_state, "final_state", (N, H, dk, dv), torch.float32, dev)
    if snapshots is None:
        snapshots = _empty(stream, nsnap, H, dk, dv, dtype=torch.float32, device=dev)
    _need(snapshots, "snapshots", (nsnap, H, dk, dv), torch.float32, dev)
    cu_arr = (ctypes.c_int32 * len(cu_list))(*cu_list)
    _check(lib.kda_prefill_noalloc(
        ctypes.byref(cfg), N, cu_arr, cu_seqlens.data_ptr(), q.data_ptr(), k.data_ptr(),
        v.data_ptr(), g.data_ptr(), beta.data_ptr(), _ptr(initial_state), out.data_ptr(),
        final_state.data_ptr(), int(snapshot_interval),
        snapshots.data_ptr() if nsnap > 0 else None, _stream(stream)))
    return out, final_state, snapshots


def decode(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
           beta: torch.Tensor, state: torch.Tensor, slots: Optional[torch.Tensor] = None,
           out_dtype: Optional[torch.dtype] = None, scale: float = 0.0,
           out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """kda_decode: one token per sequence; ``state`` [S, H, dk, dv] fp32 is
    updated in place.  q, k: [N, H, dk]; v: [N, H, dv]; g: [N, H, dk];
    beta: [N, H]; slots: [N] int32 device tensor or None (identity)."""
    lib = load()
    dev = q.device
    N, H, dk = q.shape
    dv = v.shape[2]
    for name, t, shp, dt in (("q", q, (N, H, dk), q.dtype), ("k", k, (N, H, dk), q.dtype),
                             ("v", v, (N, H, dv), q.dtype), ("g", g, (N, H, dk), torch.float32),
                             ("beta", beta, (N, H), torch.float32)):
        _need(t, name, shp, dt, dev)
    if state.dim() != 4 or tuple(state.shape[1:]) != (H, dk, dv):
        raise ValueError(f"state: shape {tuple(state.shape)} != [S, {H}, {dk}, {dv}]")
    _need(state, "state", tuple(state.shape), torch.float32, dev)
    if slots is None and state.shape[0] < N:
        raise ValueError("state has fewer rows than sequences")
    if slots is not None:
        _need(slots, "slots", (N,), torch.int32, dev)
    if out_dtype is None:
        out_dtype = out.dtype if out is not None else torch.float32
    cfg = config(H, dk, dv, q.dtype, out_dtype, scale)
    if out is None:
        out = _empty(stream, N, H, dv, dtype=out_dtype, device=dev)
    _need(out, "out", (N, H, dv), out_dtype, dev)
    _check(lib.kda_decode(ctypes.byref(cfg), N, q.data_ptr(), k.data_ptr(), v.data_ptr(),
                          g.data_ptr(), beta.data_ptr(), state.data_ptr(), _ptr(slots),
                          out.data_ptr(), _stream(stream)))
    return out


def frontend_config(H: int, dk: int, conv_width: int, in_dtype: torch.dtype,
                    out_dtype: torch.dtype = torch.bfloat16, eps: float = 1e-6) -> FrontendConfig:
    return FrontendConfig(H, dk, conv_width, _dtype_code(in_dtype), _dtype_code(out_dtype),
                          float(eps))


def qk_frontend(xq: torch.Tensor, xk: torch.Tensor, wq: torch.Tensor, wk: torch.Tensor,
                cu_seqlens: torch.Tensor, eps: float = 1e-6,
                conv_state_q: Optional[torch.Tensor] = None,
                conv_state_k: Optional[torch.Tensor] = None,
                conv_state_out_q: Optional[torch.Tensor] = None,
                conv_state_out_k: Optional[torch.Tensor] = None,
                slots: Optional[torch.Tensor] = None,
                out_dtype: Optional[torch.dtype] = None,
                cu_seqlens_host: Optional[Sequence[int]] = None,
                q_out: Optional[torch.Tensor] = None, k_out: Optional[torch.Tensor] = None,
                stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """kda_qk_frontend: short convolution -> Swish -> L2 norm of q and k.

    xq, xk: [T, H, dk] (bf16 or fp32, same dtype); wq, wk: [H*dk, W] or
    [H, dk, W] fp32 taps (tap W-1 on the current token); cu_seqlens: [N+1]
    int32 on the device.  conv_state_q/k: [S, W-1, H, dk] in the dtype of x,
    the history of each slot (None = zeros); conv_state_out_q/k: where the new
    history goes (may be the same tensors: update in place; None = not
    written).  slots: [N] int32 state rows (None = row b).  Returns (q, k)
    normalised, [T, H, dk] in out_dtype (default bf16, the dtype kda_prefill
    and kda_decode take).
    """
    lib = load()
    dev = xq.device
    T, H, dk = xq.shape
    W = int(wq.shape[-1])
    if cu_seqlens_host is None:
        cu_seqlens_host = cu_seqlens.cpu().tolist()
    cu_list = [int(x) for x in cu_seqlens_host]
    N = len(cu_list) - 1
    _need(cu_seqlens, "cu_seqlens", (N + 1,), torch.int32, dev)
    _need(xq, "xq", (T, H, dk), xq.dtype, dev)
    _need(xk, "xk", (T, H, dk), xq.dtype, dev)
    for name, w in (("wq", wq), ("wk", wk)):
        if w.numel() != H * dk * W:
            raise ValueError(f"{name}: {tuple(w.shape)} does not hold [H*dk={H * dk}, W={W}]")
        _need(w, name, tuple(w.shape), torch.float32, dev)
    if cu_list[-1] != T:
        raise ValueError(f"cu_seqlens ends at {cu_list[-1]} but xq has {T} tokens")
    states = [conv_state_q, conv_state_k, conv_state_out_q, conv_state_out_k]
    num_slots = 0
    for name, st in zip(("conv_state_q", "conv_state_k", "conv_state_out_q",
                         "conv_state_out_k"), states):
        if st is None:
            continue
        if st.dim() != 4 or tuple(st.shape[1:]) != (W - 1, H, dk):
            raise ValueError(f"{name}: shape {tuple(st.shape)} != [S, {W - 1}, {H}, {dk}]")
        _need(st, name, tuple(st.shape), xq.dtype, dev)
        if num_slots and st.shape[0] != num_slots:
            raise ValueError("all convolution states must have the same number of rows")
        num_slots = int(st.shape[0])
    if slots is not None:
        _need(slots, "slots", (N,), torch.int32, dev)
    if out_dtype is None:
        out_dtype = q_out.dtype if q_out is not None else torch.bfloat16
    cfg = frontend_config(H, dk, W, xq.dtype, out_dtype, eps)
    if q_out is None:
        q_out = _empty(stream, T, H, dk, dtype=out_dtype, device=dev)
    if k_out is None:
        k_out = _empty(stream, T, H, dk, dtype=out_dtype, device=dev)
    _need(q_out, "q_out", (T, H, dk), out_dtype, dev)
    _need(k_out, "k_out", (T, H, dk), out_dtype, dev)
    cu_arr = (ctypes.c_int32 * len(cu_list))(*cu_list)
    _check(lib.kda_qk_frontend(
        ctypes.byref(cfg), N, cu_arr, cu_seqlens.data_ptr(), xq.data_ptr(), xk.data_ptr(),
        wq.data_ptr(), wk.data_ptr(), *(_ptr(st) for st in states), _ptr(slots), num_slots,
        q_out.data_ptr(), k_out.data_ptr(), _stream(stream)))
    return q_out, k_out


MULTI_MODES = {"apply": 0, "verify": 1, "commit": 2}


def decode_multi(q: Optional[torch.Tensor], k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
                 beta: torch.Tensor, state: torch.Tensor, mode: str = "apply",
                 accepted: Optional[torch.Tensor] = None, slots: Optional[torch.Tensor] = None,
                 out_dtype: Optional[torch.dtype] = None, scale: float = 0.0,
                 out: Optional[torch.Tensor] = None, stream=None) -> Optional[torch.Tensor]:
    """kda_decode_multi: K tokens per sequence against resident states.

    k: [N, K, H, dk]; q: same (may be None in "commit"); v: [N, K, H, dv];
    g: [N, K, H, dk] fp32; beta: [N, K, H] fp32; state: [S, H, dk, dv] fp32.
    mode "apply" (outputs, state advanced by K), "verify" (outputs, state
    only read) or "commit" (the first accepted[n] tokens applied, accepted an
    [N] int32 device tensor; no output).  Returns out [N, K, H, dv] (None in
    "commit").
    """
    lib = load()
    if mode not in MULTI_MODES:
        raise ValueError(f"mode {mode!r} not in {sorted(MULTI_MODES)}")
    dev = k.device
    N, K, H, dk = k.shape
    dv = v.shape[3]
    outputs = mode != "commit"
    if outputs and q is None:
        raise ValueError(f"q is required in mode {mode!r}")
    checks = [("k", k, (N, K, H, dk), k.dtype), ("v", v, (N, K, H, dv), k.dtype),
              ("g", g, (N, K, H, dk), torch.float32), ("beta", beta, (N, K, H), torch.float32)]
    if q is not None:
        checks.append(("q", q, (N, K, H, dk), k.dtype))
    for name, t, shp, dt in checks:
        _need(t, name, shp, dt, dev)
    if state.dim() != 4 or tuple(state.shape[1:]) != (H, dk, dv):
        raise ValueError(f"state: shape {tuple(state.shape)} != [S, {H}, {dk}, {dv}]")
    _need(state, "state", tuple(state.shape), torch.float32, dev)
    if slots is None and state.shape[0] < N:
        raise ValueError("state has fewer rows than sequences")
    if slots is not None:
        _need(slots, "slots", (N,), torch.int32, dev)
    if mode == "commit":
        if accepted is None:
            raise ValueError("accepted is required in mode 'commit'")
        _need(accepted, "accepted", (N,), torch.int32, dev)
    if out_dtype is None:
        out_dtype = out.dtype if out is not None else torch.float32
    cfg = config(H, dk, dv, k.dtype, out_dtype, scale)
    if outputs:
        if out is None:
            out = _empty(stream, N, K, H, dv, dtype=out_dtype, device=dev)
        _need(out, "out", (N, K, H, dv), out_dtype, dev)
    else:
        out = None
    _check(lib.kda_decode_multi(ctypes.byref(cfg), N, K, MULTI_MODES[mode], _ptr(q), k.data_ptr(),
                                v.data_ptr(), g.data_ptr(), beta.data_ptr(), state.data_ptr(),
                                _ptr(slots), _ptr(accepted) if mode == "commit" else None,
                                _ptr(out), _stream(stream)))
    return out


def snapshot_count_at(cu_seqlens_host: Sequence[int], start_pos_host: Sequence[int],
                      interval: int) -> int:
    n = len(cu_seqlens_host) - 1
    cu = (ctypes.c_int32 * len(cu_seqlens_host))(*cu_seqlens_host)
    st = (ctypes.c_int32 * n)(*start_pos_host)
    r = load().kda_snapshot_count_at(cu, st, n, int(interval))
    if r < 0:
        raise ValueError("cu_seqlens must be non-decreasing and start positions >= 0")
    return int(r)


def pool_workspace_size(cfg: Config, num_seqs: int, total_tokens: int) -> int:
    return int(load().kda_prefill_pool_workspace_size(ctypes.byref(cfg), num_seqs, total_tokens))


def prefill_pool(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
                 beta: torch.Tensor, cu_seqlens: torch.Tensor, start_pos: torch.Tensor,
                 state_pool: torch.Tensor, slots: Optional[torch.Tensor] = None,
                 snapshot_interval: int = 0, out_dtype: Optional[torch.dtype] = None,
                 scale: float = 0.0, cu_seqlens_host: Optional[Sequence[int]] = None,
                 start_pos_host: Optional[Sequence[int]] = None,
                 out: Optional[torch.Tensor] = None, snapshots: Optional[torch.Tensor] = None,
                 workspace: Optional[torch.Tensor] = None,
                 stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """kda_prefill_pool: prefill against a pool of resident states.

    start_pos: [N] int32 device tensor, the absolute position of each
    sequence's first token (0 = fresh sequence, zero state; > 0 = its pool
    row holds the state after that many tokens).  state_pool: [S, H, dk, dv]
    fp32, rows slots[b] (or b) read and overwritten with the final states.
    Snapshots fall on absolute multiples of snapshot_interval.  Returns
    (out, snapshots)."""
    lib = load()
    dev = q.device
    T, H, dk = q.shape
    dv = v.shape[2]
    if cu_seqlens_host is None:
        cu_seqlens_host = cu_seqlens.cpu().tolist()
    if start_pos_host is None:
        start_pos_host = start_pos.cpu().tolist()
    cu_list = [int(x) for x in cu_seqlens_host]
    st_list = [int(x) for x in start_pos_host]
    N = len(cu_list) - 1
    _need(cu_seqlens, "cu_seqlens", (N + 1,), torch.int32, dev)
    _need(start_pos, "start_pos", (N,), torch.int32, dev)
    if len(st_list) != N:
        raise ValueError("start_pos_host must hold one entry per sequence")
    for name, t, shp, dt in (("q", q, (T, H, dk), q.dtype), ("k", k, (T, H, dk), q.dtype),
                             ("v", v, (T, H, dv), q.dtype), ("g", g, (T, H, dk), torch.float32),
                             ("beta", beta, (T, H), torch.float32)):
        _need(t, name, shp, dt, dev)
    if cu_list[-1] != T:
        raise ValueError(f"cu_seqlens ends at {cu_list[-1]} but q has {T} tokens")
    if state_pool.dim() != 4 or tuple(state_pool.shape[1:]) != (H, dk, dv):
        raise ValueError(f"state_pool: shape {tuple(state_pool.shape)} != [S, {H}, {dk}, {dv}]")
    _need(state_pool, "state_pool", tuple(state_pool.shape), torch.float32, dev)
    if slots is not None:
        _need(slots, "slots", (N,), torch.int32, dev)
    if out_dtype is None:
        out_dtype = out.dtype if out is not None else torch.float32
    cfg = config(H, dk, dv, q.dtype, out_dtype, scale)
    nsnap = snapshot_count_at(cu_list, st_list, snapshot_interval) if snapshot_interval > 0 else 0
    if out is None:
        out = _empty(stream, T, H, dv, dtype=out_dtype, device=dev)
    _need(out, "out", (T, H, dv), out_dtype, dev)
    if snapshots is None:
        snapshots = _empty(stream, nsnap, H, dk, dv, dtype=torch.float32, device=dev)
    _need(snapshots, "snapshots", (nsnap, H, dk, dv), torch.float32, dev)
    ws_bytes = pool_workspace_size(cfg, N, T)
    if workspace is None and ws_bytes > 0:
        workspace = _empty(stream, ws_bytes, dtype=torch.uint8, device=dev)
    cu_arr = (ctypes.c_int32 * len(cu_list))(*cu_list)
    st_arr = (ctypes.c_int32 * max(1, N))(*st_list)
    _check(lib.kda_prefill_pool(
        ctypes.byref(cfg), N, cu_arr, cu_seqlens.data_ptr(), st_arr, start_pos.data_ptr(),
        q.data_ptr(), k.data_ptr(), v.data_ptr(), g.data_ptr(), beta.data_ptr(),
        state_pool.data_ptr(), _ptr(slots), int(state_pool.shape[0]), out.data_ptr(),
        int(snapshot_interval), snapshots.data_ptr() if nsnap > 0 else None, _ptr(workspace),
        workspace.numel() if workspace is not None else 0, _stream(stream)))
    return out, snapshots


class AttnResConfig(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("num_sources", ctypes.c_int32),
                ("in_dtype", ctypes.c_int), ("out_dtype", ctypes.c_int),
                ("logit_scale", ctypes.c_float), ("eps", ctypes.c_float)]


def attnres(sources: Sequence[torch.Tensor], query: torch.Tensor,
            residual: Optional[torch.Tensor] = None, gamma: Optional[torch.Tensor] = None,
            logit_scale: float = 1.0, eps: float = 1e-6, out_dtype: Optional[torch.dtype] = None,
            h_out: Optional[torch.Tensor] = None, y_out: Optional[torch.Tensor] = None,
            want_h: bool = True, stream=None) -> Tuple[Optional[torch.Tensor], torch.Tensor]:
    """kda_attnres: softmax over the sources (logits logit_scale * <query, s>),
    weighted sum plus the residual (h), then RMSNorm with gamma (y).

    sources: M tensors [T, d] (bf16 or fp32, one dtype); query, gamma: [d]
    fp32; residual: [T, d] or None.  Returns (h or None, y)."""
    lib = load()
    M = len(sources)
    if M < 1:
        raise ValueError("at least one source")
    T, d = sources[0].shape
    dev = sources[0].device
    dt = sources[0].dtype
    for i, s in enumerate(sources):
        _need(s, f"sources[{i}]", (T, d), dt, dev)
    _need(query, "query", (d,), torch.float32, dev)
    if residual is not None:
        _need(residual, "residual", (T, d), dt, dev)
    if gamma is not None:
        _need(gamma, "gamma", (d,), torch.float32, dev)
    if out_dtype is None:
        out_dtype = y_out.dtype if y_out is not None else dt
    if y_out is None:
        y_out = _empty(stream, T, d, dtype=out_dtype, device=dev)
    _need(y_out, "y_out", (T, d), out_dtype, dev)
    if want_h and h_out is None:
        h_out = _empty(stream, T, d, dtype=out_dtype, device=dev)
    if h_out is not None:
        _need(h_out, "h_out", (T, d), out_dtype, dev)
    cfg = AttnResConfig(d, M, _dtype_code(dt), _dtype_code(out_dtype), float(logit_scale),
                        float(eps))
    ptrs = (ctypes.c_void_p * M)(*[s.data_ptr() for s in sources])
    _check(lib.kda_attnres(ctypes.byref(cfg), T, ptrs, _ptr(residual), query.data_ptr(),
                           _ptr(gamma), _ptr(h_out), y_out.data_ptr(), _stream(stream)))
    return h_out, y_out


def decode_spec_step(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
                     beta: torch.Tensor, state: torch.Tensor,
                     prev: Optional[Tuple[torch.Tensor, torch.Tensor, torch.Tensor,
                                          torch.Tensor]] = None,
                     accepted: Optional[torch.Tensor] = None,
                     slots: Optional[torch.Tensor] = None,
                     out_dtype: Optional[torch.dtype] = None, scale: float = 0.0,
                     out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """kda_decode_spec_step: commit accepted[n] tokens of the previous step
    (prev = (k, v, g, beta) of that step, [N, K, H, d] etc.) to each state,
    then verify the new draft q, k, v, g, beta [N, K, H, d]; returns its
    outputs [N, K, H, dv].  accepted None: nothing to commit."""
    lib = load()
    dev = k.device
    N, K, H, dk = k.shape
    dv = v.shape[3]
    checks = [("q", q, (N, K, H, dk), k.dtype), ("k", k, (N, K, H, dk), k.dtype),
              ("v", v, (N, K, H, dv), k.dtype), ("g", g, (N, K, H, dk), torch.float32),
              ("beta", beta, (N, K, H), torch.float32)]
    if accepted is not None:
        if prev is None:
            raise ValueError("accepted needs the previous step's (k, v, g, beta)")
        pk, pv, pg, pb = prev
        checks += [("prev_k", pk, (N, K, H, dk), k.dtype), ("prev_v", pv, (N, K, H, dv), k.dtype),
                   ("prev_g", pg, (N, K, H, dk), torch.float32),
                   ("prev_beta", pb, (N, K, H), torch.float32)]
        _need(accepted, "accepted", (N,), torch.int32, dev)
    else:
        pk = pv = pg = pb = None
    for name, t, shp, dt in checks:
        _need(t, name, shp, dt, dev)
    if state.dim() != 4 or tuple(state.shape[1:]) != (H, dk, dv):
        raise ValueError(f"state: shape {tuple(state.shape)} != [S, {H}, {dk}, {dv}]")
    _need(state, "state", tuple(state.shape), torch.float32, dev)
    if slots is None and state.shape[0] < N:
        raise ValueError("state has fewer rows than sequences")
    if slots is not None:
        _need(slots, "slots", (N,), torch.int32, dev)
    if out_dtype is None:
        out_dtype = out.dtype if out is not None else torch.float32
    cfg = config(H, dk, dv, k.dtype, out_dtype, scale)
    if out is None:
        out = _empty(stream, N, K, H, dv, dtype=out_dtype, device=dev)
    _need(out, "out", (N, K, H, dv), out_dtype, dev)
    _check(lib.kda_decode_spec_step(ctypes.byref(cfg), N, K, _ptr(pk), _ptr(pv), _ptr(pg),
                                    _ptr(pb), _ptr(accepted), q.data_ptr(), k.data_ptr(),
                                    v.data_ptr(), g.data_ptr(), beta.data_ptr(), state.data_ptr(),
                                    _ptr(slots), out.data_ptr(), _stream(stream)))
    return out
