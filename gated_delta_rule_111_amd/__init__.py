"""libkda: the Kimi Delta Attention layer (chunked prefill with state
snapshots, and single-token decode) as hand-written HIP kernels for one AMD
MI355X (gfx950) behind a C ABI (include/kda.h).

``gated_delta_rule_111_amd.kda`` is the Python binding (ctypes + torch device
memory); ``gated_delta_rule_111_amd.inputs`` draws seeded synthetic inputs.
Importing the package loads nothing; the shared library is loaded on the
first call and its absence is an error.
"""
from . import kda  # noqa: F401
from .kda import KdaError, decode, prefill, snapshot_count, workspace_size  # noqa: F401

# C-ABI names, for callers that mirror include/kda.h
kda_prefill = prefill
kda_decode = decode
