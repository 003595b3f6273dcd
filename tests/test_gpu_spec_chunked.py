"""Speculative verify, commit and the fused step for drafts of at most 8
tokens per sequence (computed in the chunked form of the recurrence) at every
head size, with gates from no decay to near-total decay and with beta = 0,
against the fp64 oracle; drafts longer than 8 tokens (computed by walking the
tokens) are checked the same way."""
import numpy as np
import pytest
import torch

from parity import TOL, slice_rel_err, state_err, to_np
from test_gpu_decode_multi import _oracle_run

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _verify_commit(inp, acc, slots, pool_size, label):
    """verify then commit on a pool through slots; both against the oracle,
    untouched slots and zero-accepted sequences unchanged."""
    from gated_delta_rule_111_amd import kda
    N, K, H, d = inp.k.shape
    gen = torch.Generator(device=DEV).manual_seed(N * 1000 + K * 10 + d)
    pool = torch.randn(pool_size, H, d, d, device=DEV, generator=gen) * 0.5
    pool0 = pool.clone()
    out = kda.decode_multi(inp.q, inp.k, inp.v, inp.g, inp.beta, pool, mode="verify",
                           slots=slots)
    torch.cuda.synchronize()
    assert torch.equal(pool, pool0), f"{label}: verify wrote a state"
    accd = torch.tensor(acc, dtype=torch.int32, device=DEV)
    kda.decode_multi(None, inp.k, inp.v, inp.g, inp.beta, pool, mode="commit",
                     accepted=accd, slots=slots)
    torch.cuda.synchronize()
    ref_o, _ = _oracle_run(inp, [K] * N, pool0, slots)
    _, ref_s = _oracle_run(inp, acc, pool0, slots)
    sl = to_np(slots)
    eo = slice_rel_err(to_np(out), ref_o, slice_axes=(0, 2))
    es = state_err(to_np(pool)[sl], ref_s)
    print(f"[{label}] verify err {eo:.2e} commit err {es:.2e}", flush=True)
    assert eo <= TOL, f"{label}: verify"
    assert es <= TOL, f"{label}: commit"
    for n, a in enumerate(acc):
        if a == 0:
            assert torch.equal(pool[sl[n]], pool0[sl[n]]), f"{label}: accepted 0 moved {n}"
    for s in sorted(set(range(pool_size)) - set(sl.tolist())):
        assert torch.equal(pool[s], pool0[s]), f"{label}: untouched slot {s} changed"


@pytest.mark.parametrize("d", [16, 32, 64, 128])
@pytest.mark.parametrize("K", [1, 3, 8])
def test_chunked_verify_commit(d, K):
    from gated_delta_rule_111_amd.inputs import multi_token_inputs
    label = f"chunked d={d} K={K}"
    print(f"[{label}]", flush=True)
    N, H = 6, 3
    inp = multi_token_inputs(N, K, H, d, d, seed=40 * d + K, state_std=0.5, device=DEV)
    acc = [(n * 5) % (K + 1) for n in range(N)]
    acc[0], acc[-1] = 0, K
    slots = torch.tensor([7, 2, 0, 5, 3, 8], dtype=torch.int32, device=DEV)
    _verify_commit(inp, acc, slots, 9, label)


@pytest.mark.parametrize("in_dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("decay_shift", [-20.0, 20.0])
def test_chunked_gate_extremes(decay_shift, in_dtype):
    """decay_shift -20: alpha ~ 1 (no forgetting); +20: alpha ~ e^-20 per
    token, so the cumulative gate underflows within the draft."""
    from gated_delta_rule_111_amd.inputs import multi_token_inputs
    label = f"gates shift={decay_shift} in={in_dtype}"
    print(f"[{label}]", flush=True)
    N, K, H, d = 5, 8, 4, 128
    inp = multi_token_inputs(N, K, H, d, d, seed=91, in_dtype=in_dtype,
                             decay_shift=decay_shift, state_std=0.5, device=DEV)
    slots = torch.tensor([1, 4, 0, 3, 2], dtype=torch.int32, device=DEV)
    _verify_commit(inp, [8, 3, 0, 1, 6], slots, 5, label)


def test_chunked_beta_zero():
    """beta = 0: no token writes the state; verify reads the decayed state
    and commit only decays it."""
    from gated_delta_rule_111_amd.inputs import multi_token_inputs
    print("[beta zero]", flush=True)
    N, K, H, d = 4, 8, 2, 64
    inp = multi_token_inputs(N, K, H, d, d, seed=17, state_std=0.5, device=DEV)
    inp = type(inp)(inp.q, inp.k, inp.v, inp.g, torch.zeros_like(inp.beta), inp.state)
    slots = torch.tensor([3, 1, 0, 2], dtype=torch.int32, device=DEV)
    _verify_commit(inp, [8, 2, 5, 1], slots, 4, "beta zero")


@pytest.mark.parametrize("d", [16, 128])
def test_step_equals_split_short_draft(d):
    """The fused step at K = 3 equals commit then verify bit for bit."""
    from gated_delta_rule_111_amd import kda
    from gated_delta_rule_111_amd.inputs import multi_token_inputs
    print(f"[step split d={d}]", flush=True)
    N, K, H = 7, 3, 2
    s_fused = torch.randn(N, H, d, d, device=DEV) * 0.1
    s_split = s_fused.clone()
    prev, acc = None, None
    for step in range(3):
        inp = multi_token_inputs(N, K, H, d, d, seed=1300 + step + d, device=DEV)
        of = kda.decode_spec_step(inp.q, inp.k, inp.v, inp.g, inp.beta, s_fused,
                                  prev=prev, accepted=acc)
        if acc is not None:
            kda.decode_multi(None, *prev, s_split, mode="commit", accepted=acc)
        osp = kda.decode_multi(inp.q, inp.k, inp.v, inp.g, inp.beta, s_split, mode="verify")
        torch.cuda.synchronize()
        assert torch.equal(of, osp), f"step {step}: outputs differ"
        assert torch.equal(s_fused, s_split), f"step {step}: states differ"
        prev = (inp.k, inp.v, inp.g, inp.beta)
        acc = torch.tensor([(n + step) % (K + 1) for n in range(N)], dtype=torch.int32,
                           device=DEV)


def test_long_draft_walk():
    """12-token drafts (more than 8: the token walk) through verify, commit
    and the fused step, against the oracle."""
    from gated_delta_rule_111_amd import kda
    from gated_delta_rule_111_amd.inputs import multi_token_inputs
    print("[long draft]", flush=True)
    N, K, H, d = 5, 12, 3, 128
    inp = multi_token_inputs(N, K, H, d, d, seed=23, state_std=0.5, device=DEV)
    slots = torch.tensor([2, 0, 4, 1, 3], dtype=torch.int32, device=DEV)
    _verify_commit(inp, [12, 0, 7, 1, 11], slots, 5, "long draft")
    # the fused step with the same draft as the previous one
    state = inp.state.clone()
    acc = torch.tensor([5, 12, 0, 9, 3], dtype=torch.int32, device=DEV)
    o = kda.decode_spec_step(inp.q, inp.k, inp.v, inp.g, inp.beta, state,
                             prev=(inp.k, inp.v, inp.g, inp.beta), accepted=acc)
    torch.cuda.synchronize()
    # reference: the accepted prefix, then the whole draft again from there
    _, mid = _oracle_run(inp, to_np(acc), inp.state)
    ref_o, _ = _oracle_run(inp, [K] * N, torch.from_numpy(mid).float())
    assert state_err(to_np(state), mid) <= TOL
    assert slice_rel_err(to_np(o), ref_o, slice_axes=(0, 2)) <= TOL
