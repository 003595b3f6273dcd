"""kda_qk_frontend (short convolution -> Swish -> L2 norm of q and k) on the
GPU against the fp64 oracle, through the C ABI.

Bars: fp32 outputs within the parity tolerance per (sequence, head) slice;
bf16 outputs correctly rounded (within half a bf16 ulp of the oracle, plus
the fp32 arithmetic's own error before the rounding); convolution states are
copies of inputs and must match bit for bit.
"""
import numpy as np
import pytest
import torch

from parity import TOL, seq_head_err, to_np

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _oracle(inp, W, eps, state_q=None, state_k=None, slots=None, num_slots=None, cu=None):
    import oracle
    cu = to_np(inp.cu_seqlens) if cu is None else cu
    sl = None if slots is None else to_np(slots)
    yq, sq = oracle.qk_frontend(to_np(inp.xq), to_np(inp.wq), cu, W, eps,
                                state=None if state_q is None else to_np(state_q),
                                slots=sl, num_slots=num_slots)
    yk, sk = oracle.qk_frontend(to_np(inp.xk), to_np(inp.wk), cu, W, eps,
                                state=None if state_k is None else to_np(state_k),
                                slots=sl, num_slots=num_slots)
    return yq, yk, sq, sk


def _bf16_rounding_err(dev, ref):
    """max over elements of |dev - ref| / (half a bf16 ulp of ref + 1e-5):
    <= 1 when every bf16 output is ref rounded to nearest, up to the fp32
    error (well under 1e-5 for unit-norm rows) ahead of the rounding."""
    dev = np.asarray(dev, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    mag = np.maximum(np.abs(ref), 2.0 ** -126)
    half_ulp = 2.0 ** (np.floor(np.log2(mag)) - 8)
    return float(np.max(np.abs(dev - ref) / (half_ulp + 1e-5))) if dev.size else 0.0


LENS = [1, 0, 37, 2, 130, 3, 0]


@pytest.mark.parametrize("dk", [16, 32, 64, 128])
@pytest.mark.parametrize("W", [1, 2, 4, 8])
@pytest.mark.parametrize("in_dtype", [torch.float32, torch.bfloat16])
def test_frontend_small(dk, W, in_dtype):
    from gated_delta_rule_111_amd import kda
    from gated_delta_rule_111_amd.inputs import frontend_inputs
    print(f"[frontend small] dk={dk} W={W} in={in_dtype}", flush=True)
    inp = frontend_inputs(LENS, 3, dk, W, seed=dk + W, in_dtype=in_dtype, device=DEV)
    q, k = kda.qk_frontend(inp.xq, inp.xk, inp.wq, inp.wk, inp.cu_seqlens, eps=1e-6,
                           out_dtype=torch.float32)
    torch.cuda.synchronize()
    yq, yk, _, _ = _oracle(inp, W, 1e-6)
    cu = to_np(inp.cu_seqlens)
    eq, ek = seq_head_err(to_np(q), yq, cu), seq_head_err(to_np(k), yk, cu)
    print(f"[frontend small] err q {eq:.2e} k {ek:.2e}", flush=True)
    assert eq <= TOL and ek <= TOL


@pytest.mark.parametrize("W", [2, 4, 8])
def test_frontend_states_slots(W):
    """History from a state pool through a slot permutation, new history to a
    second pool; empty and shorter-than-W sequences; untouched slots kept."""
    from gated_delta_rule_111_amd import kda
    from gated_delta_rule_111_amd.inputs import frontend_inputs
    print(f"[frontend states] W={W}", flush=True)
    lens = [5, 0, 1, 200, 2, 64, 7]
    S = 10
    inp = frontend_inputs(lens, 4, 64, W, seed=50 + W, num_slots=S, device=DEV)
    slots = torch.tensor([7, 2, 0, 9, 4, 1, 5], dtype=torch.int32, device=DEV)
    out_q = torch.full_like(inp.state_q, 7.0)
    out_k = torch.full_like(inp.state_k, -7.0)
    q, k = kda.qk_frontend(inp.xq, inp.xk, inp.wq, inp.wk, inp.cu_seqlens, eps=1e-6,
                           conv_state_q=inp.state_q, conv_state_k=inp.state_k,
                           conv_state_out_q=out_q, conv_state_out_k=out_k, slots=slots,
                           out_dtype=torch.float32)
    torch.cuda.synchronize()
    yq, yk, sq, sk = _oracle(inp, W, 1e-6, inp.state_q, inp.state_k, slots)
    cu = to_np(inp.cu_seqlens)
    assert seq_head_err(to_np(q), yq, cu) <= TOL
    assert seq_head_err(to_np(k), yk, cu) <= TOL
    used = to_np(slots).tolist()
    for s in used:
        assert np.array_equal(to_np(out_q[s]), sq[s]), f"q state of slot {s}"
        assert np.array_equal(to_np(out_k[s]), sk[s]), f"k state of slot {s}"
    for s in set(range(S)) - set(used):
        assert torch.all(out_q[s] == 7.0) and torch.all(out_k[s] == -7.0), f"slot {s} written"


def test_frontend_bf16_out_rounding():
    from gated_delta_rule_111_amd import kda
    from gated_delta_rule_111_amd.inputs import frontend_inputs
    print("[frontend bf16 out]", flush=True)
    inp = frontend_inputs([300, 17, 0, 900], 8, 128, 4, seed=61, num_slots=4, device=DEV)
    q, k = kda.qk_frontend(inp.xq, inp.xk, inp.wq, inp.wk, inp.cu_seqlens, eps=1e-6,
                           conv_state_q=inp.state_q, conv_state_k=inp.state_k,
                           out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    yq, yk, _, _ = _oracle(inp, 4, 1e-6, inp.state_q, inp.state_k)
    rq, rk = _bf16_rounding_err(to_np(q), yq), _bf16_rounding_err(to_np(k), yk)
    print(f"[frontend bf16 out] rounding ratio q {rq:.3f} k {rk:.3f}", flush=True)
    assert rq <= 1.0 and rk <= 1.0


def test_frontend_decode_in_place():
    """Decode steps: cu = 0, 1, ..., N, the states of a slot pool updated in
    place; a prefill of the prompt first.  Every step matches the oracle run
    over the whole history."""
    from gated_delta_rule_111_amd import kda
    from gated_delta_rule_111_amd.inputs import frontend_inputs
    print("[frontend decode]", flush=True)
    N, H, dk, W, S, steps = 48, 4, 128, 4, 64, 6
    prompt = [int(x) for x in np.random.default_rng(3).integers(0, 9, N)]
    lens = prompt + [1] * (N * steps)
    inp = frontend_inputs(lens, H, dk, W, seed=70, device=DEV)
    slots = torch.tensor(np.random.default_rng(4).permutation(S)[:N].astype(np.int32),
                         device=DEV)
    st_q = torch.zeros(S, W - 1, H, dk, dtype=torch.bfloat16, device=DEV)
    st_k = torch.zeros_like(st_q)
    T0 = sum(prompt)
    qp, kp = kda.qk_frontend(inp.xq[:T0], inp.xk[:T0], inp.wq, inp.wk,
                             inp.cu_seqlens[:N + 1].contiguous(), conv_state_out_q=st_q,
                             conv_state_out_k=st_k, slots=slots, out_dtype=torch.float32)
    step_cu = torch.arange(N + 1, dtype=torch.int32, device=DEV)
    outs_q, outs_k = [], []
    for s in range(steps):
        a = T0 + s * N
        qs, ks = kda.qk_frontend(inp.xq[a:a + N], inp.xk[a:a + N], inp.wq, inp.wk, step_cu,
                                 conv_state_q=st_q, conv_state_k=st_k,
                                 conv_state_out_q=st_q, conv_state_out_k=st_k, slots=slots,
                                 cu_seqlens_host=list(range(N + 1)), out_dtype=torch.float32)
        outs_q.append(qs)
        outs_k.append(ks)
    torch.cuda.synchronize()
    # oracle: each sequence's prompt followed by its decode tokens, in one run
    import oracle
    xq, xk = to_np(inp.xq), to_np(inp.xk)
    cu_p = np.concatenate([[0], np.cumsum(prompt)])
    for b in range(0, N, 7):
        rows = list(range(cu_p[b], cu_p[b + 1])) + [T0 + s * N + b for s in range(steps)]
        for x, w, got_p, got, st in ((xq, inp.wq, qp, outs_q, st_q), (xk, inp.wk, kp, outs_k, st_k)):
            y, new_st = oracle.qk_frontend(x[rows], to_np(w), [0, len(rows)], W, 1e-6)
            dev = np.concatenate([to_np(got_p[cu_p[b]:cu_p[b + 1]])] +
                                 [to_np(o[b:b + 1]) for o in got])
            assert seq_head_err(dev, y, [0, len(rows)]) <= TOL, f"sequence {b}"
            assert np.array_equal(to_np(st[int(slots[b])]), new_st[0]), f"state of {b}"


@pytest.mark.parametrize("W", [1, 2, 4, 8])
@pytest.mark.parametrize("in_dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("N", [1, 37])
def test_frontend_one_token_sequences(W, in_dtype, N):
    """Every sequence one token long (the decode-step launch): an odd count
    (the last wave holds fewer tokens), H*dk = 320 (a part-empty slab), history
    from one pool through permuted slots, new history to another; then the
    same call with no history (zeros) and no state written."""
    from gated_delta_rule_111_amd import kda
    from gated_delta_rule_111_amd.inputs import frontend_inputs
    print(f"[frontend one-token] W={W} in={in_dtype} N={N}", flush=True)
    S = N + 5
    inp = frontend_inputs([1] * N, 5, 64, W, seed=300 + W + N, in_dtype=in_dtype,
                          num_slots=S if W > 1 else None, device=DEV)
    cu_host = list(range(N + 1))
    cu = to_np(inp.cu_seqlens)
    if W > 1:  # W = 1 has no history
        slots = torch.tensor(np.random.default_rng(W + N).permutation(S)[:N].astype(np.int32),
                             device=DEV)
        out_q = torch.full_like(inp.state_q, 3.0)
        out_k = torch.full_like(inp.state_k, -3.0)
        q, k = kda.qk_frontend(inp.xq, inp.xk, inp.wq, inp.wk, inp.cu_seqlens, eps=1e-6,
                               conv_state_q=inp.state_q, conv_state_k=inp.state_k,
                               conv_state_out_q=out_q, conv_state_out_k=out_k, slots=slots,
                               cu_seqlens_host=cu_host, out_dtype=torch.float32)
        torch.cuda.synchronize()
        yq, yk, sq, sk = _oracle(inp, W, 1e-6, inp.state_q, inp.state_k, slots)
        assert seq_head_err(to_np(q), yq, cu) <= TOL and seq_head_err(to_np(k), yk, cu) <= TOL
        used = to_np(slots).tolist()
        for s in range(S):
            if s in used:
                assert np.array_equal(to_np(out_q[s]), sq[s]), f"q state of slot {s}"
                assert np.array_equal(to_np(out_k[s]), sk[s]), f"k state of slot {s}"
            else:
                assert torch.all(out_q[s] == 3.0) and torch.all(out_k[s] == -3.0), f"slot {s}"
    q0, k0 = kda.qk_frontend(inp.xq, inp.xk, inp.wq, inp.wk, inp.cu_seqlens, eps=1e-6,
                             cu_seqlens_host=cu_host, out_dtype=torch.float32)
    torch.cuda.synchronize()
    zq, zk, _, _ = _oracle(inp, W, 1e-6)
    assert seq_head_err(to_np(q0), zq, cu) <= TOL and seq_head_err(to_np(k0), zk, cu) <= TOL


def test_frontend_full_size():
    """T = 8192 tokens, H = 32, dk = 128, W = 4, bf16 in: the launch shape of
    the benchmark (runs of 16 tokens).  fp32 outputs against the oracle on
    every token and head."""
    from gated_delta_rule_111_amd import kda
    from gated_delta_rule_111_amd.inputs import FRONTEND_WIDTH, frontend_inputs
    print("[frontend full] T=8192 H=32 dk=128", flush=True)
    inp = frontend_inputs([8192], 32, 128, FRONTEND_WIDTH, seed=2, device=DEV)
    q, k = kda.qk_frontend(inp.xq, inp.xk, inp.wq, inp.wk, inp.cu_seqlens,
                           out_dtype=torch.float32)
    torch.cuda.synchronize()
    yq, yk, _, _ = _oracle(inp, FRONTEND_WIDTH, 1e-6)
    eq, ek = seq_head_err(to_np(q), yq, [0, 8192]), seq_head_err(to_np(k), yk, [0, 8192])
    print(f"[frontend full] err q {eq:.2e} k {ek:.2e}", flush=True)
    assert eq <= TOL and ek <= TOL


def test_frontend_long_runs_sampled():
    """40,000 tokens in 5 sequences (runs of 64 tokens, the longest the
    launch uses), bf16 out: 200 sampled tokens checked against the oracle on
    their own W-token windows."""
    from gated_delta_rule_111_amd import kda
    from gated_delta_rule_111_amd.inputs import frontend_inputs
    import oracle
    print("[frontend long] T=40000 H=32 dk=128", flush=True)
    lens = [10000, 3, 20000, 2, 9995]
    W = 4
    inp = frontend_inputs(lens, 32, 128, W, seed=80, device=DEV)
    q, k = kda.qk_frontend(inp.xq, inp.xk, inp.wq, inp.wk, inp.cu_seqlens,
                           out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    cu = np.concatenate([[0], np.cumsum(lens)])
    rng = np.random.default_rng(5)
    worst = 0.0
    xq, xk, wq, wk = (to_np(t) for t in (inp.xq, inp.xk, inp.wq, inp.wk))
    qn, kn = to_np(q), to_np(k)
    for t in sorted(rng.choice(cu[-1], 200, replace=False).tolist()):
        b = int(np.searchsorted(cu, t, side="right") - 1)
        lo = max(int(cu[b]), t - (W - 1))
        for x, w, got in ((xq, wq, qn), (xk, wk, kn)):
            y, _ = oracle.qk_frontend(x[lo:t + 1], w, [0, t + 1 - lo], W, 1e-6)
            worst = max(worst, _bf16_rounding_err(got[t], y[-1]))
    print(f"[frontend long] rounding ratio {worst:.3f}", flush=True)
    assert worst <= 1.0


def test_frontend_graph_replay():
    """The decode-step call captured in a HIP graph: each replay (with eager
    work and synchronisations between them) advances the states exactly as
    the same call made eagerly does."""
    from gated_delta_rule_111_amd import kda
    from gated_delta_rule_111_amd.inputs import frontend_inputs
    print("[frontend graph]", flush=True)
    N, H, dk, W, steps = 64, 8, 128, 4, 4
    inp = frontend_inputs([1] * N, H, dk, W, seed=90, num_slots=N, device=DEV)
    cu_host = list(range(N + 1))
    q_out = torch.empty(N, H, dk, dtype=torch.bfloat16, device=DEV)
    k_out = torch.empty_like(q_out)
    sq0, sk0 = inp.state_q.clone(), inp.state_k.clone()

    def call():
        kda.qk_frontend(inp.xq, inp.xk, inp.wq, inp.wk, inp.cu_seqlens,
                        conv_state_q=inp.state_q, conv_state_k=inp.state_k,
                        conv_state_out_q=inp.state_q, conv_state_out_k=inp.state_k,
                        cu_seqlens_host=cu_host, q_out=q_out, k_out=k_out)

    eager = []
    for _ in range(steps):
        call()
        eager.append((q_out.clone(), k_out.clone(), inp.state_q.clone(), inp.state_k.clone()))
    torch.cuda.synchronize()
    inp.state_q.copy_(sq0)
    inp.state_k.copy_(sk0)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    # capture does not run the kernels: the states are still the initial ones
    torch.cuda.synchronize()
    assert torch.equal(inp.state_q, sq0)
    for i in range(steps):
        graph.replay()
        torch.cuda.synchronize()
        junk = torch.randn(1000, device=DEV).sum().item()  # eager work between replays
        assert junk == junk
        for got, want, name in zip((q_out, k_out, inp.state_q, inp.state_k), eager[i],
                                   ("q", "k", "state_q", "state_k")):
            assert torch.equal(got, want), f"replay {i}: {name} differs from the eager call"
