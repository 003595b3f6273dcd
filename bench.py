"""libkda benchmark: the five KDA workloads on one MI355X, each with its
roofline fraction, and the fp64 oracle timed on the host beside them.

    python bench.py [--steps K] [--warmup W] [--prefill-reps R] [--no-long] ...

One JSON line is printed.  Its ``value`` is the decode rate on the workload
256 sequences x 32 heads, dk = dv = 128, bf16 q/k/v, fp32 states resident in
HBM, chained steps (a "step" advances every sequence by one token through
one KDA layer, all 32 heads).  ``configs`` holds every workload by number:
1 the tiny fp32 prefill (us per call), 2 that decode step, 3 the prefill of
B=1, H=32, T=8192 with snapshots every 1024 tokens, 4 the packed varlen
prefill of 16 sequences of 1024..32768 tokens, 5 the prefill of
T=1,048,576 with snapshots every 65,536 and the 512 decode steps that
follow it; each with ``roofline`` and ``cpu_baseline`` (the oracle on a
stated sample of the same workload).  All inputs are seeded synthetic
tensors generated on the device before timing starts.

Kernel durations come from HIP events recorded on the stream the kernels are
launched on (torch's current stream, which the binding passes to the C ABI).
``--copy-calibration MiB`` instead times a plain device copy of that size;
run under ``rocprofv3 --pmc FETCH_SIZE`` / ``WRITE_SIZE`` it gives the factor
that turns those counters into bytes.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "KDA prefill tokens/s + decode seq-steps/s; % of MFMA / HBM roofline, 1 GPU"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, TFLOP/s

# Algorithmic work per unit (the bytes a kernel must move and the flops the
# chunked method must do, independent of how the kernels are written).
#   decode, per (sequence, head, step): fp32 state read + written
#   (2 * dk * dv * 4 B) + q, k, v bf16 (3 * 256 B) + g fp32 (512 B)
#   + beta (4 B) + out fp32 (512 B)
#   prefill, per (token, head): q, k, v bf16 768 B + g 512 B + beta 4 B +
#   out fp32 512 B = 1796 B, plus snapshot and final-state bytes per call;
#   140,757 flop for the chunked form (C = 64 accounting: A, B Gram
#   triangles, the triangular solve, W and U~, the three state products, B U)
DECODE_STATE_BYTES = 2 * 128 * 128 * 4
DECODE_IO_BYTES = 3 * 128 * 2 + 128 * 4 + 4 + 128 * 4
PREFILL_BYTES_PER_TOKEN_HEAD = 1796
PREFILL_FLOP_PER_TOKEN_HEAD = 140757
STATE_BYTES = 128 * 128 * 4

TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
KERNEL_SOURCES = {
    "decode": os.path.join(ROOT, "gated_delta_rule_111_amd", "csrc", "kda_decode.hip"),
    "prefill": os.path.join(ROOT, "gated_delta_rule_111_amd", "csrc", "kda_prefill.hip"),
    "frontend": os.path.join(ROOT, "gated_delta_rule_111_amd", "csrc", "kda_frontend.hip"),
    "multi": os.path.join(ROOT, "gated_delta_rule_111_amd", "csrc", "kda_decode_multi.hip"),
    "spec": os.path.join(ROOT, "gated_delta_rule_111_amd", "csrc", "kda_spec.hip"),
    "attnres": os.path.join(ROOT, "gated_delta_rule_111_amd", "csrc", "kda_attnres.hip"),
}


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def source_hash(kind: str) -> str:
    with open(KERNEL_SOURCES[kind], "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def measured_traffic(kind: str, workload: str):
    """HBM bytes per launch from the committed rocprofv3 FETCH_SIZE/WRITE_SIZE
    runs, or None when they were taken on another version of the kernel."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f).get(kind)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_sha256_16") != source_hash(kind):
        return None
    if "workloads" in rec:
        return rec["workloads"].get(workload)
    return rec.get("bytes_per_launch") if rec.get("workload") == workload else None


def cpu_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:
        return max(1, os.cpu_count() or 1)


# ---------------------------------------------------------------------------
def bench_decode(args, torch, kda, inputs):
    w = inputs.DECODE
    dev = "cuda:0"
    log(f"[bench] decode: generating {w.decode_steps} x {w.decode_N} x {w.H} tokens")
    inp = inputs.make_decode(w, device=dev)
    state = inp.state.clone()
    out = torch.empty(w.decode_N, w.H, w.dv, dtype=torch.float32, device=dev)
    nin = inp.q.shape[0]

    def step(i):
        j = i % nin
        kda.decode(inp.q[j], inp.k[j], inp.v[j], inp.g[j], inp.beta[j], state, out=out)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for i in range(args.steps):
        step(args.warmup + i)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = e0.elapsed_time(e1)
    per_launch_s = gpu_ms / 1e3 / args.steps
    units = w.decode_N * w.H
    bytes_per_launch = units * (DECODE_STATE_BYTES + DECODE_IO_BYTES)
    achieved = bytes_per_launch / per_launch_s / 1e9
    log(f"[bench] decode: {args.steps} steps wall {wall * 1e3:.1f} ms, "
        f"events {gpu_ms:.1f} ms, {per_launch_s * 1e6:.1f} us/step, {achieved:.0f} GB/s")
    res = {
        "workload": w.name,
        "seq_steps_per_s": w.decode_N * args.steps / wall,
        "ms_per_step": wall * 1e3 / args.steps,
        "kernel_us": per_launch_s * 1e6,
        "roofline": {
            "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic("decode", w.name),
            "kernel": "decode_kernel<128,128,4,bf16,f32>",
            "bytes_per_launch": bytes_per_launch,
        },
    }
    return res, inp


def cpu_decode_baseline(inp, args):
    import numpy as np
    import oracle
    n_seq, n_steps = args.cpu_decode_seqs, args.cpu_decode_steps
    f = lambda t: t[:n_steps, :n_seq].float().cpu().numpy()
    st = inp.state[:n_seq].cpu().numpy().astype(np.float64)
    q, k, v, g, b = f(inp.q), f(inp.k), f(inp.v), f(inp.g), f(inp.beta)
    threads = cpu_threads()
    log(f"[bench] cpu oracle: decode {n_seq} seqs x {n_steps} steps on {threads} threads")
    t0 = time.perf_counter()
    oracle.decode(q, k, v, g, b, st, nthreads=threads)
    dt = time.perf_counter() - t0
    return {"value": round(n_seq * n_steps / dt, 2), "unit": "seq-steps/s", "cores": threads,
            "kind": "oracle", "seconds": round(dt, 2),
            "sample": f"first {n_steps} chained steps of the first {n_seq} of 256 sequences, "
                      "all 32 heads, fp64 token-by-token"}


# ---------------------------------------------------------------------------
def bench_prefill(torch, kda, inputs, w, reps, warmup):
    dev = "cuda:0"
    log(f"[bench] prefill {w.name}: generating inputs")
    inp = inputs.make_prefill(w, device=dev)
    T = int(inp.q.shape[0])
    cu_host = inp.cu_seqlens.cpu().tolist()
    N = len(cu_host) - 1
    nsnap = kda.snapshot_count(cu_host, w.snapshot_interval)
    out = torch.empty(T, w.H, w.dv, dtype=torch.float32, device=dev)
    fin = torch.empty(N, w.H, w.dk, w.dv, dtype=torch.float32, device=dev)
    snaps = torch.empty(nsnap, w.H, w.dk, w.dv, dtype=torch.float32, device=dev)
    cfg = kda.config(w.H, w.dk, w.dv, inp.q.dtype)
    ws = torch.empty(kda.workspace_size(cfg, N, T), dtype=torch.uint8, device=dev)

    def call():
        kda.prefill(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.cu_seqlens,
                    initial_state=inp.initial_state, snapshot_interval=w.snapshot_interval,
                    cu_seqlens_host=cu_host, out=out, final_state=fin, snapshots=snaps,
                    workspace=ws)

    for _ in range(warmup):
        call()
    _spin_up(torch, call)
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(reps):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per_call = e0.elapsed_time(e1) / 1e3 / reps
    # each call on its own between events as well: median and minimum
    singles = []
    for _ in range(reps):
        a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a0.record(stream)
        call()
        a1.record(stream)
        torch.cuda.synchronize()
        singles.append(a0.elapsed_time(a1))
    singles.sort()
    th = T * w.H
    nbytes = th * PREFILL_BYTES_PER_TOKEN_HEAD + (nsnap + N) * w.H * STATE_BYTES
    if inp.initial_state is not None:
        nbytes += N * w.H * STATE_BYTES
    flops = th * PREFILL_FLOP_PER_TOKEN_HEAD
    gbs = nbytes / per_call / 1e9
    tflops = flops / per_call / 1e12
    log(f"[bench] prefill {w.name}: {per_call * 1e3:.3f} ms/call, {T / per_call:.3e} tok/s, "
        f"{gbs:.0f} GB/s, {tflops:.1f} TFLOP/s")
    res = {
        "workload": w.name,
        "value": round(T / (wall / reps), 1),
        "unit": "tokens/s",
        "ms_per_call": round(wall * 1e3 / reps, 4),
        "kernel_ms": round(per_call * 1e3, 4),
        "kernel_ms_median": round(singles[len(singles) // 2], 4),
        "kernel_ms_min": round(singles[0], 4),
        "reps": reps,
        "dtype": "bf16 in; bf16 and fp16 MFMA (split or per-tile-scaled operands) + f32 state",
        "roofline": {
            "bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(gbs / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic("prefill", w.name),
            "kernel": "plan + prep_kernel<bf16> + scan_kernel (whole call)",
            "bytes_per_launch": nbytes,
        },
        "mfma": {
            "achieved": round(tflops, 2), "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(tflops / BF16_MFMA_PEAK_TFLOPS, 4),
            "flop_per_launch": flops,
            "attainable_frac": round(
                tflops / min(BF16_MFMA_PEAK_TFLOPS, flops / nbytes * HBM_PEAK_GBS / 1e3), 4),
        },
    }
    return res, inp, fin


def cpu_prefill_baseline(inp, tokens: int):
    import oracle
    T = min(tokens, int(inp.q.shape[0]))
    f = lambda t: t[:T].float().cpu().numpy()
    threads = cpu_threads()
    log(f"[bench] cpu oracle: prefill first {T} tokens on {threads} threads")
    t0 = time.perf_counter()
    oracle.prefill(f(inp.q), f(inp.k), f(inp.v), f(inp.g), f(inp.beta), [0, T],
                   nthreads=threads)
    dt = time.perf_counter() - t0
    return {"value": round(T / dt, 1), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "seconds": round(dt, 2),
            "sample": f"first {T} tokens of the sequence, all heads, fp64 token-by-token "
                      "(parallel over the heads only)"}


def cpu_varlen_baseline(inp, tokens_per_seq: int):
    """The oracle on the first `tokens_per_seq` tokens of each sequence of the
    varlen workload, all heads, from the workload's initial states."""
    import numpy as np
    import oracle
    cu = inp.cu_seqlens.cpu().tolist()
    parts = [(cu[b], min(cu[b + 1], cu[b] + tokens_per_seq)) for b in range(len(cu) - 1)]
    cat = lambda t: np.concatenate([t[a:e].float().cpu().numpy() for a, e in parts])
    cu2 = [0]
    for a, e in parts:
        cu2.append(cu2[-1] + e - a)
    threads = cpu_threads()
    log(f"[bench] cpu oracle: varlen first {tokens_per_seq} tokens of {len(parts)} sequences "
        f"on {threads} threads")
    q, k, v, g, b = cat(inp.q), cat(inp.k), cat(inp.v), cat(inp.g), cat(inp.beta)
    init = inp.initial_state.cpu().numpy()
    t0 = time.perf_counter()
    oracle.prefill(q, k, v, g, b, cu2, initial_state=init, nthreads=threads)
    dt = time.perf_counter() - t0
    return {"value": round(cu2[-1] / dt, 1), "unit": "tokens/s", "cores": threads,
            "kind": "oracle", "seconds": round(dt, 2),
            "sample": f"first {tokens_per_seq} tokens of each of the {len(parts)} sequences "
                      f"({cu2[-1]} tokens), all 32 heads, from the initial states, fp64 "
                      "token-by-token"}


def bench_tiny(torch, kda, inputs, reps):
    """The tiny prefill (B=1, H=1, T=64, dk=dv=16, fp32 throughout): a
    latency case.  Kernel time per call from a HIP graph of back-to-back
    calls; wall time per eager call (host checks and marshalling included).
    Algorithmic bytes: q, k, v, g fp32 in and o fp32 out (5 x 64 x 16 x 4 B),
    beta (256 B), the final state (1 KiB)."""
    dev = "cuda:0"
    w = inputs.TINY
    inp = inputs.make_prefill(w, device=dev)
    cu_host = inp.cu_seqlens.cpu().tolist()
    out = torch.empty(64, 1, 16, dtype=torch.float32, device=dev)
    fin = torch.empty(1, 1, 16, 16, dtype=torch.float32, device=dev)
    cfg = kda.config(1, 16, 16, inp.q.dtype)
    ws = torch.empty(kda.workspace_size(cfg, 1, 64), dtype=torch.uint8, device=dev)

    def call():
        kda.prefill(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.cu_seqlens,
                    cu_seqlens_host=cu_host, out=out, final_state=fin, workspace=ws)

    for _ in range(5):
        call()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        call()
    torch.cuda.synchronize()
    eager = (time.perf_counter() - t0) / reps
    _, per_call = _time_graph(torch, call, max(2, reps // 10))
    nbytes = 5 * 64 * 16 * 4 + 64 * 4 + 16 * 16 * 4
    gbs = nbytes / per_call / 1e9
    log(f"[bench] tiny prefill: {per_call * 1e6:.2f} us/call (graph), {eager * 1e6:.1f} us "
        f"eager call")
    return {"workload": w.name, "value": round(per_call * 1e6, 3), "unit": "us/call",
            "higher_is_better": False, "kernel_us": round(per_call * 1e6, 3),
            "eager_call_us": round(eager * 1e6, 2),
            "roofline": {"bound": "hbm", "achieved": round(gbs, 3), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 6),
                         "traffic": measured_traffic("prefill", w.name),
                         "kernel": "plan + prep_kernel<float> + scan_kernel (whole call)",
                         "bytes_per_launch": nbytes,
                         "note": "latency-bound: three launches for 22 KB of data"}}


def cpu_tiny_baseline(inputs, reps: int):
    import oracle
    inp = inputs.make_prefill(inputs.TINY)
    a = [t.numpy() for t in (inp.q, inp.k, inp.v, inp.g, inp.beta)]
    cu = inp.cu_seqlens.tolist()
    oracle.prefill(*a, cu, nthreads=1)
    t0 = time.perf_counter()
    for _ in range(reps):
        oracle.prefill(*a, cu, nthreads=1)
    dt = (time.perf_counter() - t0) / reps
    return {"value": round(dt * 1e6, 2), "unit": "us/call", "cores": 1, "kind": "oracle",
            "seconds": round(dt * reps, 2),
            "sample": f"the whole tiny workload, {reps} calls, fp64, one thread"}


def bench_decode_tail(torch, kda, inputs, fin, steps):
    """512 single-token decode steps of one sequence (N = 1, H = 32, d = 128)
    from the 1,048,576-token prefill's final state, tokens drawn with seed
    4 + 1000.  Kernel time per step from a HIP graph of the chained steps
    (replayed, so the state keeps advancing); wall time per eager step.
    Algorithmic bytes per step: 32 x (2 x 64 KiB of state + 1,796 B of
    token I/O)."""
    dev = "cuda:0"
    w = inputs.LONG
    d = inputs.decode_inputs(steps=steps, N=1, H=w.H, dk=w.dk, dv=w.dv, seed=w.seed + 1000,
                             device=dev)
    state = fin.clone()
    out = torch.empty(steps, 1, w.H, w.dv, dtype=torch.float32, device=dev)

    def chain():
        for s in range(steps):
            kda.decode(d.q[s], d.k[s], d.v[s], d.g[s], d.beta[s], state, out=out[s])

    chain()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    chain()
    torch.cuda.synchronize()
    eager = (time.perf_counter() - t0) / steps
    _, per_chain = _time_graph(torch, chain, 3, inner=1)
    per_step = per_chain / steps
    nbytes = w.H * (DECODE_STATE_BYTES + DECODE_IO_BYTES)
    gbs = nbytes / per_step / 1e9
    log(f"[bench] decode tail N=1: {per_step * 1e6:.2f} us/step (graph), {eager * 1e6:.1f} us "
        f"eager step")
    return {"workload": "decode-N1-H32-d128-512steps-after-1M-prefill",
            "value": round(1.0 / per_step, 1), "unit": "seq-steps/s",
            "us_per_step": round(per_step * 1e6, 3), "eager_step_us": round(eager * 1e6, 2),
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                         "traffic": measured_traffic("decode", "decode-N1-H32-d128"),
                         "kernel": "decode_kernel<128,128,4,bf16,f32>",
                         "bytes_per_launch": nbytes,
                         "note": "latency-bound: 32 workgroups move 4.25 MB per step"}}, d, state


def cpu_long_baseline(inp, tokens: int, dinp, fin_host):
    """The oracle on the first `tokens` tokens of the 1M-token sequence (all
    heads), and on the 512-step decode tail from the GPU's final state."""
    import numpy as np
    import oracle
    f = lambda t: t[:tokens].float().cpu().numpy()
    threads = cpu_threads()
    log(f"[bench] cpu oracle: long prefill first {tokens} tokens on {threads} threads")
    q, k, v, g, b = f(inp.q), f(inp.k), f(inp.v), f(inp.g), f(inp.beta)
    t0 = time.perf_counter()
    oracle.prefill(q, k, v, g, b, [0, tokens], nthreads=threads)
    dt = time.perf_counter() - t0
    h = lambda t: t.float().cpu().numpy()
    t1 = time.perf_counter()
    oracle.decode(h(dinp.q), h(dinp.k), h(dinp.v), h(dinp.g), h(dinp.beta),
                  fin_host.astype(np.float64), nthreads=threads)
    dt_dec = time.perf_counter() - t1
    steps = int(dinp.q.shape[0])
    return {"value": round(tokens / dt, 1), "unit": "tokens/s", "cores": threads,
            "kind": "oracle", "seconds": round(dt, 2),
            "sample": f"first {tokens} tokens of the 1,048,576, all 32 heads, fp64 token-by-token "
                      "(parallel over the heads only)",
            "decode_tail": {"value": round(steps / dt_dec, 1), "unit": "seq-steps/s",
                            "seconds": round(dt_dec, 3),
                            "sample": f"the {steps} decode steps (N = 1, 32 heads)"}}


# ---------------------------------------------------------------------------
def _spin_up(torch, fn, seconds=0.2):
    """Call `fn` back to back for `seconds` before a timed section: the GPU
    idles during the host-side set-up between sections (input generation,
    oracle baselines) and its clocks take a few tens of milliseconds of load
    to come back up; without this the first section after a pause runs up
    to 15% slow."""
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(8):
            fn()
        torch.cuda.synchronize()


def _time_graph(torch, fn, reps, inner=10):
    """Per-call kernel time of `fn` (which launches on torch's current
    stream) from HIP events around `reps` replays of a HIP graph holding
    `inner` back-to-back calls, so the host's own per-call cost (argument
    checks and marshalling) does not show up as idle GPU time.  Returns
    (wall seconds per call, event seconds per call)."""
    _spin_up(torch, fn)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(inner):
            fn()
    graph.replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(reps):
        graph.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    n = reps * inner
    return (time.perf_counter() - t0) / n, e0.elapsed_time(e1) / 1e3 / n


def bench_frontend(torch, kda, inputs, reps):
    """q/k front end (short convolution -> Swish -> L2 norm, W = 4) on the
    prefill shape (T = 8192, H = 32, dk = 128, bf16 in and out) and on a
    decode step of 256 sequences with their convolution states updated in
    place, each call timed inside a HIP graph (see _time_graph).  Algorithmic bytes: x read and y written once per tensor
    (2 * (2 + 2) B per channel), plus per decode sequence the W-1 history
    rows read and written (2 * 2 * (W-1) * 2 B per channel)."""
    dev = "cuda:0"
    W, H, dk = inputs.FRONTEND_WIDTH, 32, 128
    C = H * dk
    res = {}
    for name, lens, stateful in (("prefill-T8192-H32-dk128-W4", [8192], False),
                                 ("decode-N256-H32-dk128-W4", [1] * 256, True)):
        inp = inputs.frontend_inputs(lens, H, dk, W, seed=9, num_slots=len(lens) if stateful
                                     else None, device=dev)
        T = int(sum(lens))
        cu_host = inp.cu_seqlens.cpu().tolist()
        qo = torch.empty(T, H, dk, dtype=torch.bfloat16, device=dev)
        ko = torch.empty_like(qo)
        kw = dict(conv_state_q=inp.state_q, conv_state_k=inp.state_k,
                  conv_state_out_q=inp.state_q, conv_state_out_k=inp.state_k) if stateful else {}

        def call():
            kda.qk_frontend(inp.xq, inp.xk, inp.wq, inp.wk, inp.cu_seqlens,
                            cu_seqlens_host=cu_host, q_out=qo, k_out=ko, **kw)

        wall, per_call = _time_graph(torch, call, reps)
        nbytes = 2 * T * C * (2 + 2) + 2 * C * W * 4
        if stateful:
            nbytes += 2 * T * C * 2 * 2 * (W - 1)
        gbs = nbytes / per_call / 1e9
        log(f"[bench] frontend {name}: {per_call * 1e6:.1f} us/call, {gbs:.0f} GB/s")
        res[name] = {
            "tokens_per_s": round(T / wall, 1),
            "kernel_us": round(per_call * 1e6, 2),
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                         "traffic": measured_traffic("frontend", name),
                         "kernel": ("frontend_unit_kernel<4,bf16,bf16>" if stateful
                                    else "frontend_kernel<4,8,bf16,bf16>"),
                         "bytes_per_launch": nbytes},
        }
    return res


def bench_attnres(torch, kda, inputs, reps):
    """Attention Residuals aggregation at hidden 7168 with 8 sources, bf16 in
    and out, h and y written: a prefill batch of 8192 tokens and a decode
    batch of 256.  Algorithmic bytes per token: the 8 sources and the
    residual read once, h and y written once ((8 + 1 + 2) * 7168 * 2 B), plus
    the query and gamma once per launch."""
    dev = "cuda:0"
    d, M = inputs.ATTNRES_HIDDEN, inputs.ATTNRES_SOURCES
    res = {}
    for name, T in (("prefill-T8192-d7168-M8", 8192), ("decode-T256-d7168-M8", 256)):
        inp = inputs.attnres_inputs(T, d, M, seed=17, device=dev)
        h = torch.empty(T, d, dtype=torch.bfloat16, device=dev)
        y = torch.empty_like(h)

        def call():
            kda.attnres(inp.sources, inp.query, residual=inp.residual, gamma=inp.gamma,
                        h_out=h, y_out=y)

        wall, per_call = _time_graph(torch, call, reps)
        nbytes = T * d * 2 * (M + 1 + 2) + 2 * d * 4
        gbs = nbytes / per_call / 1e9
        log(f"[bench] attnres {name}: {per_call * 1e6:.1f} us/call, {gbs:.0f} GB/s")
        res[name] = {"tokens_per_s": round(T / wall, 1), "kernel_us": round(per_call * 1e6, 2),
                     "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                                  "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                                  "traffic": measured_traffic("attnres", name),
                                  "kernel": "attnres_kernel<8,bf16,bf16>",
                                  "bytes_per_launch": nbytes}}
    return res


def cpu_attnres_baseline(inputs, tokens: int):
    import oracle
    d, M = inputs.ATTNRES_HIDDEN, inputs.ATTNRES_SOURCES
    inp = inputs.attnres_inputs(tokens, d, M, seed=17)
    f = lambda t: t.float().numpy()
    log(f"[bench] cpu oracle: attnres {tokens} tokens")
    t0 = time.perf_counter()
    oracle.attnres([f(s) for s in inp.sources], f(inp.query), x=f(inp.residual),
                   gamma=f(inp.gamma))
    dt = time.perf_counter() - t0
    return {"value": round(tokens / dt, 1), "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "seconds": round(dt, 2),
            "sample": f"{tokens} tokens of the prefill shape (d = 7168, 8 sources), fp64, one thread"}


def bench_prefill_pool(torch, kda, inputs, reps, warmup):
    """Prefill against a state pool on a prefix-cache-hit shape: 8 sequences
    of 1024 tokens (T = 8192, H = 32, d = 128, bf16) continuing from seeded
    absolute positions in [1, 32768) (mostly off the 64-token grid, so each
    first chunk carries leading padding), states read from and written back
    to their pool rows, snapshots at absolute multiples of 1024.  Algorithmic
    bytes: as for prefill (1796 B per token-head) plus the initial state read
    per sequence-head, final states and snapshots."""
    dev = "cuda:0"
    lens = [1024] * 8
    N, H, d = len(lens), 32, 128
    inp = inputs.prefill_inputs(lens, H, d, d, seed=13, device=dev)
    g = torch.Generator().manual_seed(14)
    starts = torch.randint(1, 32768, (N,), generator=g, dtype=torch.int32).tolist()
    st = torch.tensor(starts, dtype=torch.int32, device=dev)
    pool0 = torch.randn(N, H, d, d, generator=torch.Generator(device=dev).manual_seed(15),
                        device=dev) * 0.02
    pool = pool0.clone()
    cu_host = inp.cu_seqlens.cpu().tolist()
    nsnap = kda.snapshot_count_at(cu_host, starts, 1024)
    out = torch.empty(sum(lens), H, d, dtype=torch.float32, device=dev)
    snaps = torch.empty(nsnap, H, d, d, dtype=torch.float32, device=dev)
    cfg = kda.config(H, d, d, inp.q.dtype)
    ws = torch.empty(kda.pool_workspace_size(cfg, N, sum(lens)), dtype=torch.uint8, device=dev)

    def call():
        kda.prefill_pool(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.cu_seqlens, st, pool,
                         snapshot_interval=1024, cu_seqlens_host=cu_host, start_pos_host=starts,
                         out=out, snapshots=snaps, workspace=ws)

    def fresh_call():
        pool.copy_(pool0)
        call()

    for _ in range(warmup):
        fresh_call()
    _spin_up(torch, fresh_call)
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    total = 0.0
    for _ in range(reps):  # each call from the same pool contents, the copy outside the timing
        pool.copy_(pool0)
        e0.record(stream)
        call()
        e1.record(stream)
        torch.cuda.synchronize()
        total += e0.elapsed_time(e1) / 1e3
    per_call = total / reps
    T = sum(lens)
    nbytes = T * H * PREFILL_BYTES_PER_TOKEN_HEAD + (2 * N + nsnap) * H * STATE_BYTES
    gbs = nbytes / per_call / 1e9
    log(f"[bench] prefill_pool 8x1024 from off-grid starts: {per_call * 1e3:.3f} ms/call, "
        f"{T / per_call:.3e} tok/s, {gbs:.0f} GB/s, {nsnap} snapshots")
    return {"workload": "pool-8x1024-H32-d128-offgrid-starts-snap1024",
            "value": round(T / per_call, 1), "unit": "tokens/s",
            "kernel_ms": round(per_call * 1e3, 4), "start_pos": starts, "snapshots": nsnap,
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                         "traffic": measured_traffic("prefill", "pool-8x1024-H32-d128-offgrid-starts-snap1024"),
                         "kernel": "plan + prep_kernel<bf16> + scan_kernel",
                         "bytes_per_launch": nbytes}}


def bench_spec(torch, kda, inputs, reps, decode_us):
    """Speculative decoding step on the decode shape (256 sequences x 32
    heads, d = 128, fp32 states): the fused step (commit the previous step's
    accepted prefix, 1 + Binomial(7, p) with mean 4.73 or 2.61, then verify
    1 + 7 new tokens), and verify and commit as separate launches; drafts of
    8 tokens take the chunked kernel (spec_kernel).  Algorithmic bytes:
    verify reads each state once (64 KiB per sequence-head) plus the 8
    tokens' inputs (q, k, v bf16, g fp32, beta) and writes their fp32
    outputs; commit reads and writes each state once plus the accepted
    tokens' k, v, g, beta; the step is the commit's bytes plus the verify's
    token inputs and outputs.  All three are bound by those bytes."""
    dev = "cuda:0"
    N, H, d, K = 256, 32, 128, inputs.SPEC_TOKENS
    inp = inputs.multi_token_inputs(N, K, H, d, d, seed=11, device=dev)
    state = inp.state.clone()
    out = torch.empty(N, K, H, d, dtype=torch.float32, device=dev)
    tok_in = 3 * d * 2 + d * 4 + 4            # q, k, v bf16 + g fp32 + beta per token-head
    tok_commit = 2 * d * 2 + d * 4 + 4        # k, v, g, beta
    res = {}
    stream = torch.cuda.current_stream()
    for name, mean in inputs.SPEC_MEAN_ACCEPTED.items():
        acc = inputs.accepted_counts(N, K, mean, seed=12, device=dev)
        n_acc = int(acc.sum().item())

        def verify():
            kda.decode_multi(inp.q, inp.k, inp.v, inp.g, inp.beta, state, mode="verify", out=out)

        def commit():
            kda.decode_multi(None, inp.k, inp.v, inp.g, inp.beta, state, mode="commit",
                             accepted=acc)

        times = {}
        for label, fn in (("verify", verify), ("commit", commit)):
            _spin_up(torch, fn)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(reps):
                fn()
            e1.record(stream)
            torch.cuda.synchronize()
            times[label] = e0.elapsed_time(e1) / 1e3 / reps
        prev = (inp.k, inp.v, inp.g, inp.beta)

        def step():
            kda.decode_spec_step(inp.q, inp.k, inp.v, inp.g, inp.beta, state, prev=prev,
                                 accepted=acc, out=out)

        _spin_up(torch, step)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            step()
        e1.record(stream)
        torch.cuda.synchronize()
        times["step"] = e0.elapsed_time(e1) / 1e3 / reps
        vb = N * H * (STATE_BYTES + K * (tok_in + d * 4))
        cb = N * H * 2 * STATE_BYTES + n_acc * H * tok_commit
        sb = cb + N * H * K * (tok_in + d * 4)
        step_s = times["step"]
        log(f"[bench] spec {name}: fused step {step_s * 1e6:.1f} us (verify "
            f"{times['verify'] * 1e6:.1f} us + commit {times['commit'] * 1e6:.1f} us apart), "
            f"{n_acc / N:.2f} accepted/seq, {n_acc / step_s:.3e} accepted tokens/s")
        res[name] = {
            "mean_accepted": round(n_acc / N, 3),
            "accepted_tokens_per_s": round(n_acc / step_s, 1),
            "speedup_vs_single_token_decode": round((n_acc / step_s) / (N / (decode_us * 1e-6)),
                                                    3),
            "step_us": round(step_s * 1e6, 2),
            "verify_us": round(times["verify"] * 1e6, 2),
            "commit_us": round(times["commit"] * 1e6, 2),
            "verify_roofline": {"bound": "hbm", "achieved": round(vb / times["verify"] / 1e9, 1),
                                "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                "frac": round(vb / times["verify"] / 1e9 / HBM_PEAK_GBS, 4),
                                "traffic": measured_traffic("spec", "verify-N256-H32-d128-K8"),
                                "kernel": "spec_kernel<verify>", "bytes_per_launch": vb},
            "commit_roofline": {"bound": "hbm", "achieved": round(cb / times["commit"] / 1e9, 1),
                                "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                "frac": round(cb / times["commit"] / 1e9 / HBM_PEAK_GBS, 4),
                                "traffic": measured_traffic("spec", f"commit-{name}"),
                                "kernel": "spec_kernel<commit>", "bytes_per_launch": cb},
            "step_roofline": {"bound": "hbm", "achieved": round(sb / step_s / 1e9, 1),
                              "peak": HBM_PEAK_GBS, "unit": "GB/s",
                              "frac": round(sb / step_s / 1e9 / HBM_PEAK_GBS, 4),
                              "traffic": measured_traffic("spec", f"step-{name}"),
                              "kernel": "spec_kernel<step>", "bytes_per_launch": sb},
        }
    return res


def cpu_frontend_baseline(inputs, tokens: int):
    import oracle
    H, dk, W = 32, 128, inputs.FRONTEND_WIDTH
    inp = inputs.frontend_inputs([tokens], H, dk, W, seed=9)
    threads = 1
    log(f"[bench] cpu oracle: frontend {tokens} tokens, q and k")
    t0 = time.perf_counter()
    for x, w in ((inp.xq, inp.wq), (inp.xk, inp.wk)):
        oracle.qk_frontend(x.float().numpy(), w.numpy(), [0, tokens], W, 1e-6)
    dt = time.perf_counter() - t0
    return {"value": round(tokens / dt, 1), "unit": "tokens/s", "cores": threads,
            "kind": "oracle", "seconds": round(dt, 2),
            "sample": f"first {tokens} tokens of the prefill shape, q and k, fp64, one thread"}


# ---------------------------------------------------------------------------
def gemm_ceiling(torch, n: int = 8192):
    """bf16 GEMM (torch.matmul, n x n x n) timed with HIP events: the
    practical dense bf16 MFMA ceiling beside the 2.5 PFLOP/s vendor peak."""
    a = torch.randn(n, n, device="cuda:0", dtype=torch.bfloat16)
    b = torch.randn(n, n, device="cuda:0", dtype=torch.bfloat16)
    for _ in range(3):
        torch.matmul(a, b)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(10):
        torch.matmul(a, b)
    e1.record(stream)
    torch.cuda.synchronize()
    sec = e0.elapsed_time(e1) / 1e3 / 10
    return round(2 * n ** 3 / sec / 1e12, 1)


def copy_calibration(torch, mib: int):
    """A plain device copy and an in-place scale of `mib` MiB, timed with HIP
    events: the practical read+write bandwidth ceiling for the decode step;
    and a bf16 GEMM for the MFMA ceiling."""
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    stream = torch.cuda.current_stream()
    res = {"copy_calibration_bytes_read": n * 4, "bytes_written": n * 4, "launches": 10}
    for name, fn in (("copy", lambda: dst.copy_(src)), ("inplace_scale", lambda: src.mul_(1.0))):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(10):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        sec = e0.elapsed_time(e1) / 1e3 / 10
        res[name + "_GBps"] = round(2 * n * 4 / sec / 1e9, 1)
    res["bf16_gemm_8192_TFLOPs"] = gemm_ceiling(torch)
    print(json.dumps(res), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000, help="timed chained decode steps")
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--prefill-reps", type=int, default=20)
    ap.add_argument("--no-long", action="store_true",
                    help="skip the 1,048,576-token prefill and its 512-step decode tail")
    ap.add_argument("--no-varlen", action="store_true",
                    help="skip the 16-sequence varlen prefill (lengths 1024..32768)")
    ap.add_argument("--no-tiny", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-frontend", action="store_true")
    ap.add_argument("--no-spec", action="store_true")
    ap.add_argument("--no-pool", action="store_true")
    ap.add_argument("--no-attnres", action="store_true")
    ap.add_argument("--cpu-attnres-tokens", type=int, default=4096)
    ap.add_argument("--cpu-frontend-tokens", type=int, default=32768)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-decode-seqs", type=int, default=128)
    ap.add_argument("--cpu-decode-steps", type=int, default=1000)
    ap.add_argument("--cpu-prefill-tokens", type=int, default=8192)
    ap.add_argument("--cpu-varlen-tokens", type=int, default=4096,
                    help="oracle sample: the first N tokens of every varlen sequence")
    ap.add_argument("--cpu-long-tokens", type=int, default=65536,
                    help="oracle sample: the first N tokens of the 1M-token sequence")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MiB")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py: the benchmark runs on one GPU only (asked for --gpus {args.gpus}, "
              f"WORLD_SIZE {world}); the KDA layer shards by sequence or head with no "
              "exchange, so a multi-GPU figure is N times the one-GPU one and is not "
              "measured here.", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible; libkda runs on an MI355X only", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    if args.copy_calibration:
        copy_calibration(torch, args.copy_calibration)
        return

    from gated_delta_rule_111_amd import inputs, kda
    kda.load()
    cpu_on = not args.no_cpu_baseline
    configs = {}

    # config 2 (the headline): decode, 256 sequences x 32 heads
    dec, dinp = bench_decode(args, torch, kda, inputs)
    configs["2"] = {"workload": dec["workload"], "value": round(dec["seq_steps_per_s"], 1),
                    "unit": "seq-steps/s", "us_per_step": round(dec["kernel_us"], 2),
                    "roofline": dec["roofline"]}
    cpu = cpu_decode_baseline(dinp, args) if cpu_on else None
    configs["2"]["cpu_baseline"] = cpu
    del dinp

    # config 1: tiny prefill (latency)
    if not args.no_tiny:
        configs["1"] = bench_tiny(torch, kda, inputs, 200)
        if cpu_on:
            configs["1"]["cpu_baseline"] = cpu_tiny_baseline(inputs, 500)

    # config 3: 8k prefill
    if not args.no_prefill:
        pre, pinp, _ = bench_prefill(torch, kda, inputs, inputs.PREFILL_8K, args.prefill_reps,
                                     max(2, args.warmup // 10))
        if cpu_on:
            pre["cpu_baseline"] = cpu_prefill_baseline(pinp, args.cpu_prefill_tokens)
        configs["3"] = pre
        del pinp

    # config 4: varlen prefill
    if not args.no_varlen:
        var, vinp, _ = bench_prefill(torch, kda, inputs, inputs.varlen_workload(), 5, 2)
        if cpu_on:
            var["cpu_baseline"] = cpu_varlen_baseline(vinp, args.cpu_varlen_tokens)
        var["seq_lens"] = list(inputs.varlen_workload().seq_lens)
        configs["4"] = var
        del vinp
        torch.cuda.empty_cache()

    # config 5: 1,048,576-token prefill, then 512 decode steps of that sequence
    if not args.no_long:
        lng, linp, lfin = bench_prefill(torch, kda, inputs, inputs.LONG, 3, 1)
        tail, tinp, _ = bench_decode_tail(torch, kda, inputs, lfin, inputs.LONG.decode_steps)
        lng["decode_tail"] = tail
        if cpu_on:
            lng["cpu_baseline"] = cpu_long_baseline(linp, args.cpu_long_tokens, tinp,
                                                    lfin.cpu().numpy())
        configs["5"] = lng
        del linp, lfin, tinp
        torch.cuda.empty_cache()

    pool = None
    if not args.no_prefill and not args.no_pool:
        pool = bench_prefill_pool(torch, kda, inputs, args.prefill_reps, 2)
    attn = None
    if not args.no_attnres:
        attn = bench_attnres(torch, kda, inputs, args.prefill_reps)
        if cpu_on:
            attn["cpu_baseline"] = cpu_attnres_baseline(inputs, args.cpu_attnres_tokens)
    spec = None
    if not args.no_spec:
        spec = bench_spec(torch, kda, inputs, args.prefill_reps, dec["kernel_us"])
    fe = None
    if not args.no_frontend:
        fe = bench_frontend(torch, kda, inputs, args.prefill_reps)
        if cpu_on:
            fe["cpu_baseline"] = cpu_frontend_baseline(inputs, args.cpu_frontend_tokens)

    line = {
        "metric": METRIC,
        "value": round(dec["seq_steps_per_s"], 1),
        "unit": "seq-steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(dec["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": dec["workload"], "num_seqs": 256, "heads": 32, "dk": 128,
                   "dv": 128, "in_dtype": "bf16", "state_dtype": "f32", "out_dtype": "f32",
                   "parallelism": "none (1 GPU)"},
        "roofline": dec["roofline"],
        "cpu_baseline": cpu,
        "decode_kernel_us": round(dec["kernel_us"], 2),
        "configs": configs,
    }
    if fe is not None:
        line["qk_frontend"] = fe
    if spec is not None:
        line["spec_decode"] = spec
    if pool is not None:
        line["prefill_pool"] = pool
    if attn is not None:
        line["attnres"] = attn
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
