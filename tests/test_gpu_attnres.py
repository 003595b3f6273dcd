"""kda_attnres (Attention Residuals aggregation: softmax over earlier block
outputs, residual add, RMSNorm) on the GPU, through the C ABI, against the
fp64 oracle.  fp32 outputs: the parity tolerance per token row; bf16
outputs: correctly rounded up to the fp32 path's own error."""
import numpy as np
import pytest
import torch

from parity import TOL, slice_rel_err, to_np

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _oracle(inp, rows=None, scale=1.0, eps=1e-6, residual=True, gamma=True):
    import oracle
    sel = (lambda t: to_np(t)) if rows is None else (lambda t: to_np(t)[rows])
    return oracle.attnres([sel(s) for s in inp.sources], to_np(inp.query),
                          x=sel(inp.residual) if residual else None,
                          gamma=to_np(inp.gamma) if gamma else None, scale=scale, eps=eps)


def _bf16_ratio(dev, ref):
    dev = np.asarray(dev, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    mag = np.maximum(np.abs(ref), 2.0 ** -126)
    half_ulp = 2.0 ** (np.floor(np.log2(mag)) - 8)
    slack = 1e-5 * np.max(np.abs(ref), axis=-1, keepdims=True)
    return float(np.max(np.abs(dev - ref) / (half_ulp + slack)))


@pytest.mark.parametrize("M", [1, 3, 8, 9, 12, 16])
@pytest.mark.parametrize("d", [16, 1040, 4096])
def test_attnres_small(M, d):
    from gated_delta_rule_111_amd import kda
    from gated_delta_rule_111_amd.inputs import attnres_inputs
    print(f"[attnres] M={M} d={d}", flush=True)
    T = 37
    inp = attnres_inputs(T, d, M, seed=M * 100 + d, in_dtype=torch.float32, device=DEV)
    h, y = kda.attnres(inp.sources, inp.query, residual=inp.residual, gamma=inp.gamma,
                       logit_scale=0.8, eps=1e-6, out_dtype=torch.float32)
    torch.cuda.synchronize()
    rh, ry = _oracle(inp, scale=0.8)
    eh = slice_rel_err(to_np(h), rh, slice_axes=(0,))
    ey = slice_rel_err(to_np(y), ry, slice_axes=(0,))
    print(f"[attnres] err h {eh:.2e} y {ey:.2e}", flush=True)
    assert eh <= TOL and ey <= TOL


def test_attnres_options_and_degenerate():
    """No residual, no gamma, h not written; a zero query (uniform weights);
    a huge logit scale (one source takes all)."""
    from gated_delta_rule_111_amd import kda
    from gated_delta_rule_111_amd.inputs import attnres_inputs
    print("[attnres options]", flush=True)
    T, d, M = 20, 7168, 8
    inp = attnres_inputs(T, d, M, seed=5, in_dtype=torch.float32, device=DEV)
    h, y = kda.attnres(inp.sources, inp.query, want_h=False, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert h is None
    _, ry = _oracle(inp, residual=False, gamma=False)
    assert slice_rel_err(to_np(y), ry, slice_axes=(0,)) <= TOL
    zq = torch.zeros_like(inp.query)
    h0, _ = kda.attnres(inp.sources, zq, residual=inp.residual, out_dtype=torch.float32)
    torch.cuda.synchronize()
    want = np.mean([to_np(s) for s in inp.sources], axis=0) + to_np(inp.residual)
    assert slice_rel_err(to_np(h0), want, slice_axes=(0,)) <= 1e-5
    hb, _ = kda.attnres(inp.sources, inp.query, residual=inp.residual, logit_scale=1e4,
                        out_dtype=torch.float32)
    torch.cuda.synchronize()
    rb, _ = _oracle(inp, scale=1e4)
    assert slice_rel_err(to_np(hb), rb, slice_axes=(0,)) <= TOL


def test_attnres_bf16_rounding():
    from gated_delta_rule_111_amd import kda
    from gated_delta_rule_111_amd.inputs import attnres_inputs
    print("[attnres bf16]", flush=True)
    T, d, M = 50, 7168, 8
    inp = attnres_inputs(T, d, M, seed=6, device=DEV)
    h, y = kda.attnres(inp.sources, inp.query, residual=inp.residual, gamma=inp.gamma)
    torch.cuda.synchronize()
    rh, ry = _oracle(inp)
    rr = max(_bf16_ratio(to_np(h), rh), _bf16_ratio(to_np(y), ry))
    print(f"[attnres bf16] rounding ratio {rr:.3f}", flush=True)
    assert rr <= 1.0


def test_attnres_full_size_sampled():
    """T = 8192 tokens, d = 7168, 8 sources, bf16: the benchmark's launch;
    96 sampled tokens against the oracle (fp32 outputs)."""
    from gated_delta_rule_111_amd import kda
    from gated_delta_rule_111_amd.inputs import ATTNRES_HIDDEN, ATTNRES_SOURCES, attnres_inputs
    print("[attnres full] T=8192 d=7168 M=8", flush=True)
    T = 8192
    inp = attnres_inputs(T, ATTNRES_HIDDEN, ATTNRES_SOURCES, seed=7, device=DEV)
    h, y = kda.attnres(inp.sources, inp.query, residual=inp.residual, gamma=inp.gamma,
                       out_dtype=torch.float32)
    torch.cuda.synchronize()
    rows = sorted(np.random.default_rng(8).choice(T, 96, replace=False).tolist()) + [0, T - 1]
    rh, ry = _oracle(inp, rows=rows)
    eh = slice_rel_err(to_np(h)[rows], rh, slice_axes=(0,))
    ey = slice_rel_err(to_np(y)[rows], ry, slice_axes=(0,))
    print(f"[attnres full] err h {eh:.2e} y {ey:.2e}", flush=True)
    assert eh <= TOL and ey <= TOL
