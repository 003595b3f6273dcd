"""Full-size workloads on the GPU: the varlen packed prefill (16 sequences of
1024..32768 tokens) and the 1,048,576-token prefill followed by 512 decode
steps, checked against the fp64 oracle on the parts the oracle can finish in
seconds, and snapshot resumption checked bit for bit against the GPU's own
uninterrupted run."""
import numpy as np
import pytest
import torch

from parity import REG, TOL, seq_head_err, state_err, to_np

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _say(msg):
    print(msg, flush=True)


def _prefill(inp, interval):
    from gated_delta_rule_111_amd import kda
    out, fin, snaps = kda.prefill(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.cu_seqlens,
                                  initial_state=inp.initial_state, snapshot_interval=interval)
    torch.cuda.synchronize()
    return out, fin, snaps


def _host(t):
    return t.float().cpu().numpy() if t.dtype == torch.bfloat16 else t.cpu().numpy()


def test_prefill_8k_resume_bit_exact():
    """T=8192, H=32: resume from snapshot 4 (after 4096 tokens) reproduces the
    second half of the uninterrupted run bit for bit."""
    from gated_delta_rule_111_amd import kda
    from gated_delta_rule_111_amd.inputs import PREFILL_8K, make_prefill
    _say("[8k resume] T=8192 H=32 snapshot 4")
    inp = make_prefill(PREFILL_8K, device=DEV)
    out, fin, snaps = _prefill(inp, 1024)
    cu = torch.tensor([0, 4096], dtype=torch.int32, device=DEV)
    sl = lambda t: t[4096:].contiguous()
    o2, f2, s2 = kda.prefill(sl(inp.q), sl(inp.k), sl(inp.v), sl(inp.g), sl(inp.beta), cu,
                             initial_state=snaps[3:4].contiguous(), snapshot_interval=1024)
    torch.cuda.synchronize()
    assert torch.equal(o2, out[4096:])
    assert torch.equal(f2, fin)
    assert torch.equal(s2, snaps[4:])


def test_varlen_config():
    """16 packed sequences, lengths uniform in [1024, 32768] (seed 3), H=32,
    d=128, initial states N(0, 0.02^2), snapshots every 4096 tokens.

    The oracle checks every token, snapshot and final state of 4 sampled heads
    across all 16 sequences; then the first 4 sequences with at least two
    snapshots are resumed from their middle snapshot in one packed call and
    compared bit for bit with the uninterrupted run."""
    from gated_delta_rule_111_amd import kda
    from gated_delta_rule_111_amd.inputs import make_prefill, varlen_workload
    import oracle
    w = varlen_workload()
    lens = list(w.seq_lens)
    _say(f"[varlen] lens {lens} total {sum(lens)}")
    inp = make_prefill(w, device=DEV)
    out, fin, snaps = _prefill(inp, w.snapshot_interval)
    cu = inp.cu_seqlens.cpu().tolist()

    heads = [0, 11, 22, 31]
    sel = lambda t: _host(t[:, heads])
    ro, rf, rs = oracle.prefill(sel(inp.q), sel(inp.k), sel(inp.v), sel(inp.g), sel(inp.beta),
                                cu, initial_state=_host(inp.initial_state[:, heads]),
                                snapshot_interval=w.snapshot_interval)
    eo = seq_head_err(_host(out[:, heads]), ro, cu)
    ef = state_err(_host(fin[:, heads]), rf)
    es = state_err(_host(snaps[:, heads]), rs)
    _say(f"[varlen] heads {heads}: out {eo:.3e} final {ef:.3e} snaps {es:.3e}")
    assert eo <= REG and ef <= REG and es <= REG

    # resume the first four sequences with >= 2 snapshots from snapshot floor(n/2)
    iv = w.snapshot_interval
    base, picks = 0, []
    for b, L in enumerate(lens):
        n = L // iv
        if n >= 2 and len(picks) < 4:
            j = n // 2
            picks.append((b, j, base + j - 1))
        base += n
    assert len(picks) == 4
    parts = [(cu[b] + j * iv, cu[b + 1]) for b, j, _ in picks]
    cat = lambda t: torch.cat([t[a:e] for a, e in parts]).contiguous()
    cu2 = [0]
    for a, e in parts:
        cu2.append(cu2[-1] + e - a)
    init2 = torch.stack([snaps[r] for _, _, r in picks]).contiguous()
    o2, f2, _ = kda.prefill(cat(inp.q), cat(inp.k), cat(inp.v), cat(inp.g), cat(inp.beta),
                            torch.tensor(cu2, dtype=torch.int32, device=DEV),
                            initial_state=init2)
    torch.cuda.synchronize()
    _say(f"[varlen] resumed sequences {[(b, j) for b, j, _ in picks]}")
    assert torch.equal(o2, cat(out)), "resumed outputs differ from the uninterrupted run"
    assert torch.equal(f2, fin[[b for b, _, _ in picks]]), "resumed final states differ"


@pytest.mark.slow
def test_long_context_config():
    """B=1, H=32, d=128, T=1,048,576 (seed 4), snapshots every 65,536 tokens.

    Checked against the oracle: every output of the first 65,536 tokens and
    snapshot 1; the first 4,096 outputs of every later segment, with the
    oracle started from the GPU's own fp32 snapshot at that segment's start;
    the whole last segment and the final state.  Then 512 single-token decode
    steps from the GPU's final state, all against the oracle."""
    from gated_delta_rule_111_amd import kda
    from gated_delta_rule_111_amd.inputs import LONG, decode_inputs, make_prefill
    import oracle
    iv, seg_check = LONG.snapshot_interval, 4096
    _say("[long] generating T=1048576 H=32 inputs")
    inp = make_prefill(LONG, device=DEV)
    T = int(inp.q.shape[0])
    out, fin, snaps = _prefill(inp, iv)
    assert snaps.shape[0] == T // iv
    assert bool(torch.isfinite(out).all()) and bool(torch.isfinite(fin).all())

    def ora(a, e, init):
        sl = lambda t: _host(t[a:e])
        return oracle.prefill(sl(inp.q), sl(inp.k), sl(inp.v), sl(inp.g), sl(inp.beta),
                              [0, e - a], initial_state=init)

    ro, rf, _ = ora(0, iv, None)
    eo = seq_head_err(_host(out[:iv]), ro, [0, iv])
    es = state_err(_host(snaps[0:1]), rf)
    _say(f"[long] first segment: out {eo:.3e} snapshot 1 {es:.3e}")
    assert eo <= REG and es <= REG
    worst = 0.0
    nseg = T // iv
    for j in range(1, nseg):
        a = j * iv
        e = a + (iv if j == nseg - 1 else seg_check)
        init = _host(snaps[j - 1:j]).astype(np.float64)
        ro, rf, _ = ora(a, e, init)
        err = seq_head_err(_host(out[a:e]), ro, [0, e - a])
        worst = max(worst, err)
        if j == nseg - 1:
            ef = state_err(_host(fin), rf)
            _say(f"[long] last segment: out {err:.3e} final {ef:.3e}")
            assert ef <= REG
    _say(f"[long] segments 1..{nseg - 1} from GPU snapshots: worst out {worst:.3e}")
    assert worst <= REG
    assert torch.equal(snaps[-1], fin[0]), "last snapshot is the final state"

    # 512 decode steps (N = 1) from the GPU final state; tokens drawn with seed 4 + 1000
    dinp = decode_inputs(steps=512, N=1, H=32, dk=128, dv=128, seed=LONG.seed + 1000,
                         device=DEV)
    state = fin.clone()
    outs = torch.empty(512, 1, 32, 128, device=DEV)
    for s in range(512):
        kda.decode(dinp.q[s], dinp.k[s], dinp.v[s], dinp.g[s], dinp.beta[s], state, out=outs[s])
    torch.cuda.synchronize()
    h = lambda t: _host(t)
    rdo, rds = oracle.decode(h(dinp.q), h(dinp.k), h(dinp.v), h(dinp.g), h(dinp.beta),
                             _host(fin).astype(np.float64))
    from parity import slice_rel_err
    edo = slice_rel_err(_host(outs), rdo, slice_axes=(1, 2))
    eds = state_err(_host(state), rds)
    _say(f"[long] 512 decode steps: out {edo:.3e} state {eds:.3e}")
    assert edo <= REG and eds <= REG
