"""kda_decode_multi (several tokens per sequence: apply, speculative verify,
commit of the accepted prefix) on the GPU, through the C ABI, against the
fp64 oracle: a sequence's K tokens are a K-token prefill from its resident
state, so verify's outputs are that prefill's outputs and commit's state is
the final state of the prefill of the accepted prefix."""
import numpy as np
import pytest
import torch

from parity import TOL, slice_rel_err, state_err, to_np

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _oracle_run(inp, lens, state0, slots=None):
    """Oracle prefill of the first lens[n] tokens of each sequence from its
    state (through slots).  Returns (out [N, K, H, dv] with zeros past
    lens[n], final [N, H, dk, dv])."""
    import oracle
    N, K, H, dk = inp.k.shape
    dv = inp.v.shape[3]
    rows = [n * K + j for n in range(N) for j in range(int(lens[n]))]
    f = lambda t: to_np(t).reshape(N * K, *t.shape[2:])[rows]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    st = to_np(state0).astype(np.float64)
    init = st if slots is None else st[to_np(slots)]
    o, fin, _ = oracle.prefill(f(inp.q), f(inp.k), f(inp.v), f(inp.g), f(inp.beta), cu,
                               initial_state=init)
    out = np.zeros((N * K, H, dv))
    out[rows] = o
    return out.reshape(N, K, H, dv), fin


@pytest.mark.parametrize("d", [16, 32, 64, 128])
def test_multi_apply_equals_chained_decode(d):
    """apply with K tokens is K single-token decode calls, bit for bit."""
    from gated_delta_rule_111_amd import kda
    from gated_delta_rule_111_amd.inputs import multi_token_inputs
    print(f"[multi apply] d={d}", flush=True)
    N, K, H = 5, 6, 3
    inp = multi_token_inputs(N, K, H, d, d, seed=200 + d, device=DEV)
    s_multi = inp.state.clone()
    out = kda.decode_multi(inp.q, inp.k, inp.v, inp.g, inp.beta, s_multi, mode="apply")
    s_chain = inp.state.clone()
    outs = [kda.decode(inp.q[:, j].contiguous(), inp.k[:, j].contiguous(),
                       inp.v[:, j].contiguous(), inp.g[:, j].contiguous(),
                       inp.beta[:, j].contiguous(), s_chain) for j in range(K)]
    torch.cuda.synchronize()
    assert torch.equal(s_multi, s_chain)
    assert torch.equal(out, torch.stack(outs, dim=1))


@pytest.mark.parametrize("K", [1, 8, 20])
@pytest.mark.parametrize("in_dtype", [torch.float32, torch.bfloat16])
def test_multi_verify_matches_oracle(K, in_dtype):
    from gated_delta_rule_111_amd import kda
    from gated_delta_rule_111_amd.inputs import multi_token_inputs
    print(f"[multi verify] K={K} in={in_dtype}", flush=True)
    N, H, d = 6, 4, 128
    inp = multi_token_inputs(N, K, H, d, d, seed=300 + K, in_dtype=in_dtype, state_std=0.5,
                             device=DEV)
    pool = torch.randn(9, H, d, d, device=DEV) * 0.5
    slots = torch.tensor([4, 0, 8, 2, 7, 5], dtype=torch.int32, device=DEV)
    pool0 = pool.clone()
    out = kda.decode_multi(inp.q, inp.k, inp.v, inp.g, inp.beta, pool, mode="verify",
                           slots=slots)
    torch.cuda.synchronize()
    assert torch.equal(pool, pool0), "verify wrote a state"
    ref, _ = _oracle_run(inp, [K] * N, pool0, slots)
    err = slice_rel_err(to_np(out), ref, slice_axes=(0, 2))
    print(f"[multi verify] err {err:.2e}", flush=True)
    assert err <= TOL


def test_multi_commit_matches_oracle():
    from gated_delta_rule_111_amd import kda
    from gated_delta_rule_111_amd.inputs import multi_token_inputs
    print("[multi commit]", flush=True)
    N, K, H, d = 7, 8, 4, 128
    inp = multi_token_inputs(N, K, H, d, d, seed=41, state_std=0.5, device=DEV)
    acc = [3, 0, 8, 1, 5, 8, 2]
    pool = torch.randn(10, H, d, d, device=DEV) * 0.5
    slots = torch.tensor([9, 1, 3, 0, 6, 4, 8], dtype=torch.int32, device=DEV)
    pool0 = pool.clone()
    r = kda.decode_multi(None, inp.k, inp.v, inp.g, inp.beta, pool, mode="commit",
                         accepted=torch.tensor(acc, dtype=torch.int32, device=DEV), slots=slots)
    torch.cuda.synchronize()
    assert r is None
    _, fin = _oracle_run(inp, acc, pool0, slots)
    sl = to_np(slots)
    err = state_err(to_np(pool)[sl], fin)
    print(f"[multi commit] state err {err:.2e}", flush=True)
    assert err <= TOL
    assert torch.equal(pool[1], pool0[1]), "accepted 0 changed the state"
    for s in (2, 5, 7):
        assert torch.equal(pool[s], pool0[s]), f"untouched slot {s} changed"
    # out-of-range counts are clamped to [0, K]
    pool2 = pool0.clone()
    kda.decode_multi(None, inp.k, inp.v, inp.g, inp.beta, pool2, mode="commit",
                     accepted=torch.tensor([-4, 0, 99, 0, 0, 0, 0], dtype=torch.int32,
                                           device=DEV), slots=slots)
    torch.cuda.synchronize()
    _, fin2 = _oracle_run(inp, [0, 0, 8, 0, 0, 0, 0], pool0, slots)
    assert torch.equal(pool2[9], pool0[9])
    assert state_err(to_np(pool2)[[3]], fin2[[2]]) <= TOL


def test_speculative_steps():
    """Four steps of verify (1 + 7 tokens) then commit of a random accepted
    prefix; the accepted outputs and the final states match the oracle run
    over each sequence's accepted token stream."""
    from gated_delta_rule_111_amd import kda
    from gated_delta_rule_111_amd.inputs import accepted_counts, multi_token_inputs
    print("[multi spec steps]", flush=True)
    N, K, H, d, steps = 16, 8, 4, 128, 4
    state = torch.randn(N, H, d, d, device=DEV) * 0.02
    state0 = state.clone()
    streams = []
    for s in range(steps):
        inp = multi_token_inputs(N, K, H, d, d, seed=500 + s, device=DEV)
        acc = accepted_counts(N, K, 4.73, seed=600 + s, device=DEV)
        out = kda.decode_multi(inp.q, inp.k, inp.v, inp.g, inp.beta, state, mode="verify")
        kda.decode_multi(None, inp.k, inp.v, inp.g, inp.beta, state, mode="commit", accepted=acc)
        streams.append((inp, to_np(acc), out))
    torch.cuda.synchronize()
    import oracle
    for n in (0, 5, 11, 15):
        toks = {key: [] for key in ("q", "k", "v", "g", "beta")}
        outs = []
        for inp, acc, out in streams:
            a = int(acc[n])
            for key in toks:
                toks[key].append(to_np(getattr(inp, key)[n, :a]))
            outs.append(to_np(out[n, :a]))
        cat = {key: np.concatenate(v) for key, v in toks.items()}
        L = len(cat["k"])
        o, fin, _ = oracle.prefill(cat["q"], cat["k"], cat["v"], cat["g"], cat["beta"], [0, L],
                                   initial_state=to_np(state0[n:n + 1]).astype(np.float64))
        assert slice_rel_err(np.concatenate(outs), o, slice_axes=(1,)) <= TOL, f"outputs of {n}"
        assert state_err(to_np(state[n:n + 1]), fin) <= TOL, f"state of {n}"


def test_multi_full_size():
    """256 sequences x 32 heads, d = 128, 1 + 7 tokens: verify then commit
    (mean 4.73 accepted); 8 sampled sequences against the oracle."""
    from gated_delta_rule_111_amd import kda
    from gated_delta_rule_111_amd.inputs import SPEC_TOKENS, accepted_counts, multi_token_inputs
    print("[multi full] N=256 H=32 d=128 K=8", flush=True)
    N, K, H, d = 256, SPEC_TOKENS, 32, 128
    inp = multi_token_inputs(N, K, H, d, d, seed=7, device=DEV)
    acc = accepted_counts(N, K, 4.73, seed=8, device=DEV)
    state = inp.state.clone()
    out = kda.decode_multi(inp.q, inp.k, inp.v, inp.g, inp.beta, state, mode="verify")
    kda.decode_multi(None, inp.k, inp.v, inp.g, inp.beta, state, mode="commit", accepted=acc)
    torch.cuda.synchronize()
    seqs = [0, 1, 77, 128, 200, 255]
    sub = type(inp)(*(t[seqs] for t in (inp.q, inp.k, inp.v, inp.g, inp.beta)),
                    inp.state[seqs])
    ref_o, _ = _oracle_run(sub, [K] * len(seqs), inp.state[seqs])
    _, ref_s = _oracle_run(sub, to_np(acc)[seqs], inp.state[seqs])
    eo = slice_rel_err(to_np(out[seqs]), ref_o, slice_axes=(0, 2))
    es = state_err(to_np(state[seqs]), ref_s)
    print(f"[multi full] verify err {eo:.2e} commit err {es:.2e}", flush=True)
    assert eo <= TOL and es <= TOL


def test_spec_step_equals_commit_then_verify():
    """The fused step (commit the previous step's accepted tokens, verify the
    new draft) gives the commit-then-verify results bit for bit."""
    from gated_delta_rule_111_amd import kda
    from gated_delta_rule_111_amd.inputs import accepted_counts, multi_token_inputs
    print("[spec step fused]", flush=True)
    N, K, H, d = 12, 8, 4, 128
    s_fused = torch.randn(N + 3, H, d, d, device=DEV) * 0.05
    s_split = s_fused.clone()
    slots = torch.tensor(np.random.default_rng(2).permutation(N + 3)[:N].astype(np.int32),
                         device=DEV)
    prev, acc = None, None
    for step in range(4):
        inp = multi_token_inputs(N, K, H, d, d, seed=700 + step, device=DEV)
        of = kda.decode_spec_step(inp.q, inp.k, inp.v, inp.g, inp.beta, s_fused,
                                  prev=prev, accepted=acc, slots=slots)
        if acc is not None:
            kda.decode_multi(None, prev[0], prev[1], prev[2], prev[3], s_split, mode="commit",
                             accepted=acc, slots=slots)
        osp = kda.decode_multi(inp.q, inp.k, inp.v, inp.g, inp.beta, s_split, mode="verify",
                               slots=slots)
        torch.cuda.synchronize()
        assert torch.equal(of, osp), f"step {step}: outputs differ"
        assert torch.equal(s_fused, s_split), f"step {step}: states differ"
        prev = (inp.k, inp.v, inp.g, inp.beta)
        acc = accepted_counts(N, K, 2.61 if step % 2 else 4.73, seed=800 + step, device=DEV)
        if step == 2:
            acc[0] = 0  # nothing accepted for one sequence
            acc[1] = K


def test_spec_step_chain_matches_oracle():
    """Five fused steps and a last commit: the accepted outputs and final
    states equal the oracle run over each sequence's accepted tokens."""
    from gated_delta_rule_111_amd import kda
    from gated_delta_rule_111_amd.inputs import accepted_counts, multi_token_inputs
    import oracle
    print("[spec step chain]", flush=True)
    N, K, H, d, steps = 10, 8, 4, 128, 5
    state = torch.randn(N, H, d, d, device=DEV) * 0.02
    state0 = state.clone()
    prev, acc, streams = None, None, []
    for s in range(steps):
        inp = multi_token_inputs(N, K, H, d, d, seed=900 + s, device=DEV)
        out = kda.decode_spec_step(inp.q, inp.k, inp.v, inp.g, inp.beta, state, prev=prev,
                                   accepted=acc)
        acc = accepted_counts(N, K, 4.73, seed=950 + s, device=DEV)
        prev = (inp.k, inp.v, inp.g, inp.beta)
        streams.append((inp, to_np(acc), out))
    kda.decode_multi(None, *prev, state, mode="commit", accepted=acc)
    torch.cuda.synchronize()
    for n in (0, 4, 9):
        toks = {key: [] for key in ("q", "k", "v", "g", "beta")}
        outs = []
        for inp, a_np, out in streams:
            a = int(a_np[n])
            for key in toks:
                toks[key].append(to_np(getattr(inp, key)[n, :a]))
            outs.append(to_np(out[n, :a]))
        cat = {key: np.concatenate(v) for key, v in toks.items()}
        L = len(cat["k"])
        o, fin, _ = oracle.prefill(cat["q"], cat["k"], cat["v"], cat["g"], cat["beta"], [0, L],
                                   initial_state=to_np(state0[n:n + 1]).astype(np.float64))
        assert slice_rel_err(np.concatenate(outs), o, slice_axes=(1,)) <= TOL, f"outputs of {n}"
        assert state_err(to_np(state[n:n + 1]), fin) <= TOL, f"state of {n}"
