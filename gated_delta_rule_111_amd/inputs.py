"""Seeded synthetic inputs for the KDA layer (prefill and decode).

This module holds no part of the recurrence: it only draws random tensors in
a fixed order so that the HIP path and the fp64 oracle can be fed identical
values.  Nothing here is a model weight or a dataset item.

Recipe (every tensor is drawn with ``torch.randn``/``torch.rand`` from one
``torch.Generator`` seeded with the workload's seed, in this order, one block
of at most ``block_tokens`` tokens at a time: q, k, v, beta-logits, g-logits;
initial states last):

* q, k ~ N(0, 1) in fp32, L2-normalised per (token, head) in fp32, then
  rounded to the input dtype (bf16 with round-to-nearest-even, or kept fp32);
* v ~ N(0, 1), rounded to the input dtype;
* beta = sigmoid(N(0, 1) + beta_shift) in fp32 (beta_shift 0 for every
  workload; +4 gives beta ~ 0.98, the full-write regime of the stress runs);
* g = log(alpha) = -softplus(N(0, 1) + decay_shift) in fp32, so
  alpha = exp(-softplus(N(0, 1) + decay_shift)) per key channel;
* initial states ~ N(0, state_std^2) in fp32 (std, not variance), or absent.

Varlen lengths are integers uniform in [lo, hi] inclusive, drawn first from a
CPU generator with the workload seed.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import List, Optional, Sequence

import torch


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _unit_rows(x: torch.Tensor) -> torch.Tensor:
    return x / torch.linalg.vector_norm(x, dim=-1, keepdim=True)


@dataclass
class PrefillInputs:
    q: torch.Tensor          # [T, H, dk]  in_dtype
    k: torch.Tensor          # [T, H, dk]  in_dtype
    v: torch.Tensor          # [T, H, dv]  in_dtype
    g: torch.Tensor          # [T, H, dk]  fp32, log(alpha) <= 0
    beta: torch.Tensor       # [T, H]      fp32
    cu_seqlens: torch.Tensor  # [N+1] int32, on the same device
    initial_state: Optional[torch.Tensor]  # [N, H, dk, dv] fp32 or None

    @property
    def seq_lens(self) -> List[int]:
        cu = self.cu_seqlens.cpu().tolist()
        return [cu[i + 1] - cu[i] for i in range(len(cu) - 1)]


@dataclass
class DecodeInputs:
    q: torch.Tensor      # [steps, N, H, dk] in_dtype
    k: torch.Tensor      # [steps, N, H, dk] in_dtype
    v: torch.Tensor      # [steps, N, H, dv] in_dtype
    g: torch.Tensor      # [steps, N, H, dk] fp32
    beta: torch.Tensor   # [steps, N, H]     fp32
    state: torch.Tensor  # [N, H, dk, dv]    fp32


def varlen_lengths(num: int, lo: int, hi: int, seed: int) -> List[int]:
    """Integer lengths uniform in [lo, hi] inclusive (CPU generator)."""
    g = _gen(seed, "cpu")
    return torch.randint(lo, hi + 1, (num,), generator=g).tolist()


def _draw_token_block(gen, n, H, dk, dv, in_dtype, decay_shift, device, beta_shift=0.0):
    q = _unit_rows(torch.randn(n, H, dk, generator=gen, device=device)).to(in_dtype)
    k = _unit_rows(torch.randn(n, H, dk, generator=gen, device=device)).to(in_dtype)
    v = torch.randn(n, H, dv, generator=gen, device=device).to(in_dtype)
    beta = torch.sigmoid(torch.randn(n, H, generator=gen, device=device) + beta_shift)
    g = -torch.nn.functional.softplus(
        torch.randn(n, H, dk, generator=gen, device=device) + decay_shift)
    return q, k, v, g, beta


def prefill_inputs(seq_lens: Sequence[int], H: int, dk: int, dv: int,
                   seed: int, in_dtype=torch.bfloat16, decay_shift: float = 2.0,
                   state_std: Optional[float] = None, device="cpu",
                   block_tokens: int = 65536, beta_shift: float = 0.0) -> PrefillInputs:
    """Packed varlen prefill inputs; sequence b occupies rows
    [cu[b], cu[b+1]) of every [T, H, *] tensor."""
    gen = _gen(seed, device)
    T = int(sum(seq_lens))
    q = torch.empty(T, H, dk, dtype=in_dtype, device=device)
    k = torch.empty(T, H, dk, dtype=in_dtype, device=device)
    v = torch.empty(T, H, dv, dtype=in_dtype, device=device)
    g = torch.empty(T, H, dk, dtype=torch.float32, device=device)
    beta = torch.empty(T, H, dtype=torch.float32, device=device)
    for t0 in range(0, T, block_tokens):
        n = min(block_tokens, T - t0)
        bq, bk, bv, bg, bb = _draw_token_block(gen, n, H, dk, dv, in_dtype,
                                               decay_shift, device, beta_shift)
        q[t0:t0 + n] = bq
        k[t0:t0 + n] = bk
        v[t0:t0 + n] = bv
        g[t0:t0 + n] = bg
        beta[t0:t0 + n] = bb
    cu = [0]
    for L in seq_lens:
        cu.append(cu[-1] + int(L))
    cu_t = torch.tensor(cu, dtype=torch.int32, device=device)
    init = None
    if state_std is not None:
        init = torch.randn(len(seq_lens), H, dk, dv, generator=gen,
                           device=device) * float(state_std)
    return PrefillInputs(q, k, v, g, beta, cu_t, init)


def decode_inputs(steps: int, N: int, H: int, dk: int, dv: int, seed: int,
                  in_dtype=torch.bfloat16, decay_shift: float = 2.0,
                  state_std: float = 0.02, device="cpu") -> DecodeInputs:
    """All ``steps`` tokens of every sequence pre-drawn as [steps, N, H, *]."""
    gen = _gen(seed, device)
    q, k, v, g, beta = _draw_token_block(gen, steps * N, H, dk, dv, in_dtype,
                                         decay_shift, device)
    shp = (steps, N, H)
    state = torch.randn(N, H, dk, dv, generator=gen, device=device) * float(state_std)
    return DecodeInputs(q.view(*shp, dk), k.view(*shp, dk), v.view(*shp, dv),
                        g.view(*shp, dk), beta.view(*shp), state)


# ---------------------------------------------------------------------------
# The five workloads (sizes, dtypes and distributions).  The pages describe
# a 1,048,576-token context ("Moonshot releases Kimi K3 report", section "The
# architecture is built around inference cost") and a serve with
# --max-num-seqs 512 --max-model-len 32768 ("Day-0 vLLM support for Kimi K3",
# section "Deployment"); head count and head dim are this library's choice.
# ---------------------------------------------------------------------------
@dataclass(frozen=True)
class Workload:
    name: str
    kind: str                 # "prefill" | "decode" | "prefill+decode"
    seed: int
    H: int
    dk: int
    dv: int
    in_dtype: torch.dtype
    decay_shift: float
    seq_lens: tuple = ()
    state_std: Optional[float] = None
    snapshot_interval: int = 0
    decode_N: int = 0
    decode_steps: int = 0


TINY = Workload("tiny-prefill-T64-H1-d16-fp32", "prefill", 0, 1, 16, 16,
                torch.float32, 0.0, seq_lens=(64,))
DECODE = Workload("decode-N256-H32-d128-1000steps", "decode", 1, 32, 128, 128,
                  torch.bfloat16, 2.0, state_std=0.02, decode_N=256,
                  decode_steps=1000)
PREFILL_8K = Workload("prefill-B1-T8192-H32-d128-snap1024", "prefill", 2, 32,
                      128, 128, torch.bfloat16, 2.0, seq_lens=(8192,),
                      snapshot_interval=1024)
VARLEN_NUM, VARLEN_LO, VARLEN_HI, VARLEN_SEED = 16, 1024, 32768, 3
LONG_T = 1 << 20
LONG = Workload("long-prefill-B1-T1048576-H32-d128-snap65536+decode512",
                "prefill+decode", 4, 32, 128, 128, torch.bfloat16, 2.0,
                seq_lens=(LONG_T,), snapshot_interval=65536, decode_N=1,
                decode_steps=512)


def varlen_workload() -> Workload:
    lens = tuple(varlen_lengths(VARLEN_NUM, VARLEN_LO, VARLEN_HI, VARLEN_SEED))
    return Workload("varlen-16seq-1024..32768-H32-d128-snap4096", "prefill",
                    VARLEN_SEED, 32, 128, 128, torch.bfloat16, 2.0,
                    seq_lens=lens, state_std=0.02, snapshot_interval=4096)


def make_prefill(w: Workload, device="cpu", seq_lens=None) -> PrefillInputs:
    return prefill_inputs(seq_lens if seq_lens is not None else w.seq_lens,
                          w.H, w.dk, w.dv, w.seed, w.in_dtype, w.decay_shift,
                          w.state_std, device)


def make_decode(w: Workload, device="cpu", steps=None, N=None) -> DecodeInputs:
    return decode_inputs(steps if steps is not None else w.decode_steps,
                         N if N is not None else w.decode_N, w.H, w.dk, w.dv,
                         w.seed, w.in_dtype, w.decay_shift,
                         w.state_std if w.state_std is not None else 0.02,
                         device)


# ---------------------------------------------------------------------------
# q/k front end (short convolution -> Swish -> L2 norm).  The pages give no
# width or initialisation; the taps are drawn like a freshly initialised
# depthwise convolution, U(-1/sqrt(W), 1/sqrt(W)) (fan-in W), and the raw q/k
# (the projections' outputs) and any convolution history as N(0, 1).
# Drawing order: xq, xk, wq, wk, state_q, state_k.
# ---------------------------------------------------------------------------
FRONTEND_WIDTH = 4


@dataclass
class FrontendInputs:
    xq: torch.Tensor                 # [T, H, dk] in_dtype
    xk: torch.Tensor                 # [T, H, dk] in_dtype
    wq: torch.Tensor                 # [H*dk, W]  fp32
    wk: torch.Tensor                 # [H*dk, W]  fp32
    cu_seqlens: torch.Tensor         # [N+1] int32
    state_q: Optional[torch.Tensor]  # [S, W-1, H, dk] in_dtype or None
    state_k: Optional[torch.Tensor]


def frontend_inputs(seq_lens: Sequence[int], H: int, dk: int, W: int, seed: int,
                    in_dtype=torch.bfloat16, num_slots: Optional[int] = None,
                    device="cpu") -> FrontendInputs:
    """Packed varlen front-end inputs; with num_slots, N(0,1) histories for
    that many state rows."""
    gen = _gen(seed, device)
    T = int(sum(seq_lens))
    xq = torch.randn(T, H, dk, generator=gen, device=device).to(in_dtype)
    xk = torch.randn(T, H, dk, generator=gen, device=device).to(in_dtype)
    bound = 1.0 / float(W) ** 0.5
    wq = (torch.rand(H * dk, W, generator=gen, device=device) * 2 - 1) * bound
    wk = (torch.rand(H * dk, W, generator=gen, device=device) * 2 - 1) * bound
    sq = sk = None
    if num_slots is not None:
        sq = torch.randn(num_slots, W - 1, H, dk, generator=gen, device=device).to(in_dtype)
        sk = torch.randn(num_slots, W - 1, H, dk, generator=gen, device=device).to(in_dtype)
    cu = [0]
    for L in seq_lens:
        cu.append(cu[-1] + int(L))
    cu_t = torch.tensor(cu, dtype=torch.int32, device=device)
    return FrontendInputs(xq, xk, wq, wk, cu_t, sq, sk)


# ---------------------------------------------------------------------------
# Speculative decoding: K = 1 + 7 tokens per sequence per step ("Kimi K3
# technical FAQ", question "What does it take to serve K3 today?": 7 draft
# tokens).  Accepted tokens per step = 1 + Binomial(7, p) with p chosen for
# the mean the pages report ("Moonshot releases Kimi K3 report...", section
# "A third party tripled single-user decoding speed"): 4.73 for coding, 2.61
# for creative writing.  The tensors of a step are drawn as for decode and
# laid out [N, K, H, d] (sequence-major).
# ---------------------------------------------------------------------------
SPEC_TOKENS = 8
SPEC_MEAN_ACCEPTED = {"coding": 4.73, "creative": 2.61}


def accepted_counts(N: int, K: int, mean: float, seed: int, device="cpu") -> torch.Tensor:
    """[N] int32 in [1, K]: 1 + Binomial(K - 1, (mean - 1) / (K - 1))."""
    g = _gen(seed, "cpu")
    p = (float(mean) - 1.0) / (K - 1)
    draws = torch.rand(N, K - 1, generator=g) < p
    return (1 + draws.sum(dim=1)).to(torch.int32).to(device)


def multi_token_inputs(N: int, K: int, H: int, dk: int, dv: int, seed: int,
                       in_dtype=torch.bfloat16, decay_shift: float = 2.0,
                       state_std: float = 0.02, device="cpu") -> DecodeInputs:
    """decode_inputs with the token axis second: q, k [N, K, H, dk] etc.;
    the state stays [N, H, dk, dv]."""
    d = decode_inputs(K, N, H, dk, dv, seed, in_dtype, decay_shift, state_std, device)
    t = lambda x: x.transpose(0, 1).contiguous()
    return DecodeInputs(t(d.q), t(d.k), t(d.v), t(d.g), t(d.beta), d.state)


# ---------------------------------------------------------------------------
# Attention Residuals aggregation: M sources (the embedding and earlier block
# outputs) and the residual ~ N(0, 1) rounded to the input dtype; the
# pseudo-query ~ N(0, 1/d) (logits of order one); gamma = 1 + 0.1 N(0, 1).
# Hidden size 7168 ("Kimi K3 technical FAQ", question "What does the
# architecture actually look like?": the router's latent is half the 7,168
# hidden size).  Drawing order: sources, residual, query, gamma.
# ---------------------------------------------------------------------------
ATTNRES_HIDDEN = 7168
ATTNRES_SOURCES = 8


@dataclass
class AttnResInputs:
    sources: List[torch.Tensor]  # M x [T, d]
    residual: torch.Tensor       # [T, d]
    query: torch.Tensor          # [d] fp32
    gamma: torch.Tensor          # [d] fp32


def attnres_inputs(T: int, d: int, M: int, seed: int, in_dtype=torch.bfloat16,
                   device="cpu") -> AttnResInputs:
    gen = _gen(seed, device)
    src = [torch.randn(T, d, generator=gen, device=device).to(in_dtype) for _ in range(M)]
    x = torch.randn(T, d, generator=gen, device=device).to(in_dtype)
    w = torch.randn(d, generator=gen, device=device) / float(d) ** 0.5
    gamma = 1 + 0.1 * torch.randn(d, generator=gen, device=device)
    return AttnResInputs(src, x, w, gamma)
