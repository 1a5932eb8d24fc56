"""Seeded synthetic inputs for the gated delta-rule mixer.

This module only draws random numbers and applies the caller-side input
activations that sit *outside* the mixer core: L2 normalisation of q and k
(the feature map is the identity inside the mixer, per the "How it works"
section of the linear-attention wiki page, which notes that many modern
variants use an identity feature map), beta = sigmoid(noise) and
log(alpha) = -softplus(noise + shift) (the gates live in (0,1), per the Gated
DeltaNet section of the linear-attention blog post).  It holds none of the
recurrence's arithmetic, so both the fp64 oracle and the HIP path can consume
what it returns without sharing any of the method's code.

Draw order for every workload (one ``torch.Generator`` seeded once):
q, k, v, beta-noise, alpha-noise, then the initial state.

``raw_inputs`` draws inputs for the library's optional input-side prologue
instead: q and k un-normalised (each token scaled by a log-normal factor, so
norms spread over two orders of magnitude) and the gates as the raw
pre-activations b and a (beta = sigmoid(b), alpha = sigmoid(a) on the
library's side); it applies no activation at all.

Tensors are returned on the CPU unless a generator device is asked for
(``chunked_inputs``, ``decode_stream``).  q, k, v are cast to the workload's
dtype (bf16 or fp32); beta, log_alpha and states are always fp32.
"""
from __future__ import annotations

import dataclasses

import torch

ALPHA_NONE, ALPHA_SCALAR, ALPHA_CHANNEL = 0, 1, 2
MODE_NAMES = {ALPHA_NONE: "none", ALPHA_SCALAR: "scalar", ALPHA_CHANNEL: "channel"}

# Gate shifts: log alpha = -softplus(N(0,1) + shift).
SHIFT_SCALAR = 2.0   # Gated DeltaNet workloads (mean log alpha about -2.13)
SHIFT_CHANNEL = 3.0  # channel-wise (Kimi-style) workload (mean about -3.05)


@dataclasses.dataclass(frozen=True)
class ChunkedWorkload:
    name: str
    B: int
    H: int
    L: int
    dk: int
    dv: int
    C: int
    dtype: torch.dtype
    mode: int
    seed: int
    s0_std: float = 0.0  # 0 => no initial state (zero)

    @property
    def tokens(self) -> int:
        return self.B * self.L


@dataclasses.dataclass(frozen=True)
class DecodeWorkload:
    name: str
    N: int
    H: int
    dk: int
    dv: int
    steps: int
    dtype: torch.dtype
    mode: int
    seed: int
    s0_std: float = 0.02


# The five workloads the measurements are quoted on.
DELTANET_FP32 = ChunkedWorkload("deltanet_fp32_B1_H2_L256_d64", 1, 2, 256, 64, 64, 64,
                                torch.float32, ALPHA_NONE, 1)
GDN_BF16 = ChunkedWorkload("gdn_bf16_B8_H8_L2048_d128", 8, 8, 2048, 128, 128, 64,
                           torch.bfloat16, ALPHA_SCALAR, 2)
KDA_BF16 = ChunkedWorkload("kda_bf16_B4_H16_L4096_d128", 4, 16, 4096, 128, 128, 64,
                           torch.bfloat16, ALPHA_CHANNEL, 3)
SWEEP_BL = ((32, 2048), (8, 8192), (2, 32768), (1, 65536))
GDN_SWEEP = tuple(
    ChunkedWorkload(f"gdn_bf16_sweep_B{b}_H16_L{l}_d128", b, 16, l, 128, 128, 64,
                    torch.bfloat16, ALPHA_SCALAR, 4)
    for b, l in SWEEP_BL)
DECODE_BF16 = DecodeWorkload("gdn_decode_bf16_N256_H16_d128", 256, 16, 128, 128, 1024,
                             torch.bfloat16, ALPHA_SCALAR, 5)


@dataclasses.dataclass(frozen=True)
class VarlenWorkload:
    name: str
    N: int          # sequences packed per call
    H: int
    T: int          # packed tokens per head
    dk: int
    dv: int
    C: int
    dtype: torch.dtype
    mode: int
    seed: int

    @property
    def tokens(self) -> int:
        return self.T


# The headline's 16 384 tokens per head (8 x 2048) as a packed prefill batch of
# 16 prompts of mixed length.
VARLEN_GDN_BF16 = VarlenWorkload("gdn_bf16_varlen_N16_H8_T16384_d128", 16, 8, 16384, 128, 128, 64,
                                 torch.bfloat16, ALPHA_SCALAR, 6)


def varlen_lengths(N: int, T: int, seed: int) -> list[int]:
    """N sequence lengths summing to T: log-uniform draws over [64, 4096]
    scaled to the total (each at least 1)."""
    g = torch.Generator().manual_seed(seed)
    raw = torch.exp(torch.empty(N).uniform_(4.1589, 8.3178, generator=g))   # ln 64 .. ln 4096
    lens = [max(1, int(x)) for x in (raw / raw.sum() * T)]
    lens[int(torch.argmax(raw))] += T - sum(lens)
    return lens


def _l2norm(x: torch.Tensor) -> torch.Tensor:
    n = x.norm(dim=-1, keepdim=True)
    return x / torch.clamp(n, min=1e-6)


def _gate_shift(mode: int) -> float:
    return SHIFT_CHANNEL if mode == ALPHA_CHANNEL else SHIFT_SCALAR


def chunked_inputs(B: int, H: int, L: int, dk: int, dv: int, dtype: torch.dtype,
                   mode: int, seed: int, s0_std: float = 0.0,
                   alpha_shift: float | None = None, device="cpu") -> dict:
    """Inputs for one chunked-forward call, drawn in the fixed order.

    Returns a dict with q, k [B,H,L,dk], v [B,H,L,dv] (``dtype``), beta
    [B,H,L] fp32, log_alpha (None | [B,H,L] | [B,H,L,dk]) fp32 and S0
    (None | [B,H,dv,dk] fp32).  ``device`` places the generator and the
    tensors (the CPU by default; a GPU generator draws a different stream
    from the same recipe, for timing runs too large to draw on the host).
    """
    g = torch.Generator(device=device).manual_seed(seed)
    rnd = lambda *shape: torch.randn(*shape, generator=g, device=device)
    q = rnd(B, H, L, dk)
    k = rnd(B, H, L, dk)
    v = rnd(B, H, L, dv)
    beta = torch.sigmoid(rnd(B, H, L))
    shift = _gate_shift(mode) if alpha_shift is None else alpha_shift
    if mode == ALPHA_NONE:
        log_alpha = None
    elif mode == ALPHA_SCALAR:
        log_alpha = -torch.nn.functional.softplus(rnd(B, H, L) + shift)
    elif mode == ALPHA_CHANNEL:
        log_alpha = -torch.nn.functional.softplus(rnd(B, H, L, dk) + shift)
    else:
        raise ValueError(f"unknown alpha mode {mode}")
    S0 = None
    if s0_std > 0:
        S0 = rnd(B, H, dv, dk) * s0_std
    return dict(q=_l2norm(q).to(dtype).contiguous(), k=_l2norm(k).to(dtype).contiguous(),
                v=v.to(dtype).contiguous(), beta=beta.contiguous(),
                log_alpha=None if log_alpha is None else log_alpha.contiguous(),
                S0=None if S0 is None else S0.contiguous())


def workload_inputs(w: ChunkedWorkload, device="cpu") -> dict:
    return chunked_inputs(w.B, w.H, w.L, w.dk, w.dv, w.dtype, w.mode, w.seed, w.s0_std,
                          device=device)


def decode_inputs(N: int, H: int, dk: int, dv: int, steps: int, dtype: torch.dtype,
                  mode: int, seed: int, s0_std: float = 0.02,
                  alpha_shift: float | None = None) -> dict:
    """Inputs for ``steps`` consecutive decode steps over N sequences.

    q, k [steps,N,H,dk], v [steps,N,H,dv] (``dtype``); beta [steps,N,H];
    log_alpha None | [steps,N,H] | [steps,N,H,dk]; S0 [N,H,dv,dk] fp32.
    """
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(steps, N, H, dk, generator=g)
    k = torch.randn(steps, N, H, dk, generator=g)
    v = torch.randn(steps, N, H, dv, generator=g)
    beta = torch.sigmoid(torch.randn(steps, N, H, generator=g))
    shift = _gate_shift(mode) if alpha_shift is None else alpha_shift
    if mode == ALPHA_NONE:
        log_alpha = None
    elif mode == ALPHA_SCALAR:
        log_alpha = -torch.nn.functional.softplus(torch.randn(steps, N, H, generator=g) + shift)
    else:
        log_alpha = -torch.nn.functional.softplus(
            torch.randn(steps, N, H, dk, generator=g) + shift)
    S0 = torch.randn(N, H, dv, dk, generator=g) * s0_std
    return dict(q=_l2norm(q).to(dtype).contiguous(), k=_l2norm(k).to(dtype).contiguous(),
                v=v.to(dtype).contiguous(), beta=beta.contiguous(),
                log_alpha=None if log_alpha is None else log_alpha.contiguous(),
                S0=S0.contiguous())


def decode_stream(N: int, H: int, dk: int, dv: int, dtype: torch.dtype, mode: int, seed: int,
                  s0_std: float = 0.02, alpha_shift: float | None = None, device="cpu"):
    """Inputs of consecutive decode steps drawn one step at a time, for runs
    too long to hold every step's inputs at once.

    Returns (S0, steps): S0 [N,H,dv,dk] fp32, and an endless iterator of
    per-step dicts with q, k [N,H,dk], v [N,H,dv] (``dtype``), beta [N,H]
    and log_alpha (None | [N,H] | [N,H,dk]), all on ``device``.  One
    generator on ``device``, seeded once; draw order: S0, then per step q, k,
    v, beta-noise, alpha-noise.  Same distributions as ``decode_inputs``."""
    g = torch.Generator(device=device).manual_seed(seed)
    rnd = lambda *shape: torch.randn(*shape, generator=g, device=device)
    S0 = (rnd(N, H, dv, dk) * s0_std).contiguous()
    shift = _gate_shift(mode) if alpha_shift is None else alpha_shift

    def steps():
        while True:
            q = rnd(N, H, dk)
            k = rnd(N, H, dk)
            v = rnd(N, H, dv)
            beta = torch.sigmoid(rnd(N, H))
            if mode == ALPHA_NONE:
                la = None
            elif mode == ALPHA_SCALAR:
                la = -torch.nn.functional.softplus(rnd(N, H) + shift)
            else:
                la = -torch.nn.functional.softplus(rnd(N, H, dk) + shift)
            yield dict(q=_l2norm(q).to(dtype).contiguous(), k=_l2norm(k).to(dtype).contiguous(),
                       v=v.to(dtype).contiguous(), beta=beta.contiguous(),
                       log_alpha=None if la is None else la.contiguous())

    return S0, steps()


def decode_workload_inputs(w: DecodeWorkload, steps: int | None = None) -> dict:
    return decode_inputs(w.N, w.H, w.dk, w.dv, w.steps if steps is None else steps,
                         w.dtype, w.mode, w.seed, w.s0_std)


def raw_inputs(lead: tuple, L: int | None, dk: int, dv: int, dtype: torch.dtype, mode: int,
               seed: int, s0_std: float = 0.0, alpha_shift: float | None = None,
               raw_qk: bool = True, raw_gates: bool = True) -> dict:
    """Inputs for the input-side prologue: q, k [*lead, (L,) dk], v
    [*lead, (L,) dv] in ``dtype``; beta, log_alpha (None | [*lead, (L)] |
    [*lead, (L,) dk]) fp32; S0 (None | [*lead, dv, dk]).  L = None drops the
    token axis (decode).

    raw_qk: q and k un-normalised, each token scaled by a log-normal factor;
    else L2-normalised as in ``chunked_inputs``.
    raw_gates: beta = b and log_alpha = a are the pre-activations, with
    a = -(N(0,1) + shift) so that sigmoid(a) has the decay distribution of the
    activated workloads; else beta = sigmoid(b), log alpha = -softplus(-a) as
    in ``chunked_inputs`` (a call that asks only for the normalisation must
    get gates in their domain)."""
    g = torch.Generator().manual_seed(seed)
    tok = tuple(lead) + (() if L is None else (L,))
    scale = lambda: torch.exp(torch.randn(tok + (1,), generator=g))   # log-normal per token
    q = torch.randn(tok + (dk,), generator=g) * scale()
    k = torch.randn(tok + (dk,), generator=g) * scale()
    v = torch.randn(tok + (dv,), generator=g)
    b = torch.randn(tok, generator=g)
    shift = _gate_shift(mode) if alpha_shift is None else alpha_shift
    if mode == ALPHA_NONE:
        a = None
    elif mode == ALPHA_SCALAR:
        a = -(torch.randn(tok, generator=g) + shift)
    elif mode == ALPHA_CHANNEL:
        a = -(torch.randn(tok + (dk,), generator=g) + shift)
    else:
        raise ValueError(f"unknown alpha mode {mode}")
    S0 = None
    if s0_std > 0:
        S0 = torch.randn(tuple(lead) + (dv, dk), generator=g) * s0_std
    if not raw_qk:
        q, k = _l2norm(q), _l2norm(k)
    if not raw_gates:
        b = torch.sigmoid(b)
        a = None if a is None else -torch.nn.functional.softplus(-a)
    return dict(q=q.to(dtype).contiguous(), k=k.to(dtype).contiguous(),
                v=v.to(dtype).contiguous(), beta=b.contiguous(),
                log_alpha=None if a is None else a.contiguous(),
                S0=None if S0 is None else S0.contiguous())
