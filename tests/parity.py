"""Parity metric and helpers shared by the GPU tests.

Parity bar (floating point): per (sequence, head) slice, the maximum
absolute difference divided by the maximum magnitude of the oracle's values
in that slice, max|x - y| / max|y|, must be <= 2e-3; any NaN or Inf fails.
The max over slices is what is compared.  A relative error per element is
ill-posed where outputs cross zero, so it is not the criterion.
"""
import numpy as np
import torch

TOL = 2e-3

# Regression gate of the prefill tests: half the bar.  Every prefill result
# measured on the MI355X (ragged and varlen batches, every head size and
# decay regime, the exact-write and no-forgetting runs, the full-size
# workloads) has stayed at or below 5.7e-4, and the kernels are deterministic
# (fixed reduction orders, no atomics), so a change that roughly doubles an
# error fails here while still inside the bar.
REG = 1e-3


def to_np(t):
    if isinstance(t, torch.Tensor):
        return t.detach().float().cpu().numpy() if t.dtype == torch.bfloat16 \
            else t.detach().cpu().numpy()
    return np.asarray(t)


def slice_rel_err(x, y, slice_axes):
    """max over slices of max|x-y| / max|y|, a slice being everything except
    ``slice_axes`` (the axes that index slices).  Returns inf if x has a
    non-finite value."""
    x = np.asarray(x, dtype=np.float64)
    y = np.asarray(y, dtype=np.float64)
    assert x.shape == y.shape, (x.shape, y.shape)
    if not np.all(np.isfinite(x)):
        return float("inf")
    red = tuple(i for i in range(x.ndim) if i not in slice_axes)
    num = np.max(np.abs(x - y), axis=red) if red else np.abs(x - y)
    den = np.max(np.abs(y), axis=red) if red else np.abs(y)
    den = np.where(den > 0, den, 1.0)
    return float(np.max(num / den)) if num.size else 0.0


def seq_head_err(out_gpu, out_ref, cu):
    """Per (sequence, head) error of packed outputs [T, H, dv]."""
    worst = 0.0
    x = np.asarray(out_gpu, dtype=np.float64)
    y = np.asarray(out_ref, dtype=np.float64)
    for b in range(len(cu) - 1):
        s, e = int(cu[b]), int(cu[b + 1])
        if e > s:
            worst = max(worst, slice_rel_err(x[s:e], y[s:e], slice_axes=(1,)))
    return worst


def state_err(s_gpu, s_ref):
    """Per (row, head) error of states [N, H, dk, dv]."""
    return slice_rel_err(s_gpu, s_ref, slice_axes=(0, 1))
