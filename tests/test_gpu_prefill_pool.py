"""kda_prefill_pool (prefill against a pool of resident states, with
absolute start positions and snapshots at absolute multiples of the
interval) on the GPU, through the C ABI, against the fp64 oracle."""
import numpy as np
import pytest
import torch

from parity import REG, TOL, seq_head_err, state_err, to_np

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _run(inp, starts, pool, slots, interval, out_dtype=torch.float32):
    from gated_delta_rule_111_amd import kda
    st = torch.tensor(starts, dtype=torch.int32, device=DEV)
    out, snaps = kda.prefill_pool(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.cu_seqlens, st, pool,
                                  slots=slots, snapshot_interval=interval, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return out, snaps


def _oracle(inp, starts, pool0, slots, interval):
    import oracle
    f = lambda t: to_np(t)
    sl = list(range(len(starts))) if slots is None else to_np(slots).tolist()
    init = np.stack([to_np(pool0[s]).astype(np.float64) if st > 0 else
                     np.zeros(pool0.shape[1:]) for s, st in zip(sl, starts)])
    return oracle.prefill(f(inp.q), f(inp.k), f(inp.v), f(inp.g), f(inp.beta),
                          to_np(inp.cu_seqlens), initial_state=init,
                          snapshot_interval=interval, start_pos=starts)


@pytest.mark.parametrize("interval", [64, 192])
@pytest.mark.parametrize("in_dtype", [torch.bfloat16, torch.float32])
def test_pool_matches_oracle(interval, in_dtype):
    """Start positions on and off the 64-token grid (pads of 0..63 rows),
    empty and one-token sequences, a slot permutation with unused rows."""
    from gated_delta_rule_111_amd.inputs import prefill_inputs
    print(f"[pool] interval={interval} in={in_dtype}", flush=True)
    lens = [300, 0, 1, 63, 64, 65, 200, 130]
    starts = [0, 17, 4095, 37, 64, 1000, 191, 0]
    H, d = 4, 128
    inp = prefill_inputs(lens, H, d, d, seed=31, in_dtype=in_dtype, device=DEV)
    S = 11
    pool = torch.randn(S, H, d, d, device=DEV) * 0.3
    slots = torch.tensor([9, 2, 0, 5, 7, 1, 10, 4], dtype=torch.int32, device=DEV)
    pool0 = pool.clone()
    out, snaps = _run(inp, starts, pool, slots, interval)
    ro, rf, rs = _oracle(inp, starts, pool0, slots, interval)
    cu = to_np(inp.cu_seqlens)
    eo = seq_head_err(to_np(out), ro, cu)
    sl = to_np(slots)
    ef = state_err(to_np(pool)[sl], rf)
    es = state_err(to_np(snaps), rs) if rs.shape[0] else 0.0
    print(f"[pool] out {eo:.2e} final {ef:.2e} snaps {es:.2e} ({rs.shape[0]} snapshots)",
          flush=True)
    assert snaps.shape[0] == rs.shape[0]
    assert eo <= REG and ef <= REG and es <= REG
    for r in set(range(S)) - set(sl.tolist()):
        assert torch.equal(pool[r], pool0[r]), f"untouched row {r} changed"
    # the empty sequence keeps its row (its start is > 0: the state is read back)
    assert torch.equal(pool[2], pool0[2])


def test_pool_resume_from_snapshot_is_bit_exact():
    """Prefill 1000 tokens from position 0 with snapshots every 128; resume
    from the snapshot at 384 (a pool row) with start position 384: outputs
    and final state equal the uninterrupted run bit for bit."""
    from gated_delta_rule_111_amd.inputs import prefill_inputs
    print("[pool resume]", flush=True)
    H, d, L, P = 4, 128, 1000, 384
    inp = prefill_inputs([L], H, d, d, seed=33, device=DEV)
    pool = torch.zeros(2, H, d, d, device=DEV)
    out_full, snaps = _run(inp, [0], pool, None, 128)
    j = P // 128 - 1
    pool2 = torch.zeros(3, H, d, d, device=DEV)
    pool2[2] = snaps[j]
    sub = type(inp)(inp.q[P:].contiguous(), inp.k[P:].contiguous(), inp.v[P:].contiguous(),
                    inp.g[P:].contiguous(), inp.beta[P:].contiguous(),
                    torch.tensor([0, L - P], dtype=torch.int32, device=DEV), None)
    out_rest, snaps_rest = _run(sub, [P], pool2, torch.tensor([2], dtype=torch.int32, device=DEV),
                                128)
    assert torch.equal(out_rest, out_full[P:])
    assert torch.equal(pool2[2], pool[0])
    assert torch.equal(snaps_rest, snaps[j + 1:])


def test_pool_at_zero_equals_prefill():
    """All start positions 0, rows b: the same launches as kda_prefill with
    zero initial states, bit for bit."""
    from gated_delta_rule_111_amd import kda
    from gated_delta_rule_111_amd.inputs import prefill_inputs
    print("[pool zero]", flush=True)
    lens = [150, 64, 0, 333]
    H, d = 2, 128
    inp = prefill_inputs(lens, H, d, d, seed=34, device=DEV)
    pool = torch.full((4, H, d, d), 5.0, device=DEV)
    out_p, snaps_p = _run(inp, [0] * 4, pool, None, 64)
    out, fin, snaps = kda.prefill(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.cu_seqlens,
                                  snapshot_interval=64)
    torch.cuda.synchronize()
    assert torch.equal(out_p, out) and torch.equal(pool, fin) and torch.equal(snaps_p, snaps)


def test_pool_split_off_grid():
    """A 700-token sequence split at 250 (off the chunk grid): the second
    call starts at 250 from the first call's final state; both calls together
    match the oracle's single run (snapshots at 256, 512)."""
    from gated_delta_rule_111_amd.inputs import prefill_inputs
    import oracle
    print("[pool split]", flush=True)
    H, d, L, m = 4, 128, 700, 250
    inp = prefill_inputs([L], H, d, d, seed=35, device=DEV)
    pool = torch.zeros(1, H, d, d, device=DEV)
    part = lambda a, b: type(inp)(inp.q[a:b].contiguous(), inp.k[a:b].contiguous(),
                                  inp.v[a:b].contiguous(), inp.g[a:b].contiguous(),
                                  inp.beta[a:b].contiguous(),
                                  torch.tensor([0, b - a], dtype=torch.int32, device=DEV), None)
    o1, s1 = _run(part(0, m), [0], pool, None, 256)
    o2, s2 = _run(part(m, L), [m], pool, None, 256)
    assert s1.shape[0] == 0 and s2.shape[0] == 2
    f = lambda t: to_np(t)
    ro, rf, rs = oracle.prefill(f(inp.q), f(inp.k), f(inp.v), f(inp.g), f(inp.beta), [0, L],
                                snapshot_interval=256)
    assert seq_head_err(np.concatenate([to_np(o1), to_np(o2)]), ro, [0, L]) <= REG
    assert state_err(to_np(pool), rf) <= REG
    assert state_err(to_np(s2), rs) <= REG
