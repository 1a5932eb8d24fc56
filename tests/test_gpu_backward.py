"""GPU parity of the chunked backward (gdr_bwd_chunked): every gradient
against the fp64 oracle's reverse mode on the same rounded inputs
(max relative error per (batch, head): 1e-4 for fp32, 2e-2 for bf16)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import gated_delta_rule_88_amd as gdr
import gdr_inputs as gi
import oracle
from gpu_common import TOL, rel_err

pytestmark = pytest.mark.gpu

MODES = [gi.ALPHA_NONE, gi.ALPHA_SCALAR, gi.ALPHA_CHANNEL]
DTYPES = [torch.float32, torch.bfloat16]
NAMES = ("dq", "dk", "dv", "dbeta", "dlog_alpha", "dS0")


def grads_inputs(B, H, L, dk, dv, dt, mode, seed, s0_std=0.1, final=True):
    x = gi.chunked_inputs(B, H, L, dk, dv, dt, mode, seed=seed, s0_std=s0_std)
    g = torch.Generator().manual_seed(seed + 7)
    x["dO"] = torch.randn(B, H, L, dv, generator=g).to(dt)
    x["dS_final"] = torch.randn(B, H, dv, dk, generator=g) * 0.1 if final else None
    return x


def run_bwd(x, C=64):
    d = {k: (None if v is None else v.cuda()) for k, v in x.items()}
    g = gdr.gdr_bwd_chunked(d["q"], d["k"], d["v"], d["beta"], d["log_alpha"], d["S0"], d["dO"],
                            d["dS_final"], C)
    torch.cuda.synchronize()
    return {k: (None if v is None else v.float().cpu().numpy()) for k, v in g.items()}


def oracle_bwd(x):
    return oracle.backward(x["q"], x["k"], x["v"], x["beta"], x["log_alpha"], x["S0"], x["dO"],
                           x["dS_final"])


def check(g, r, tol):
    for name in NAMES:
        if r[name] is None:
            assert g[name] is None
            continue
        got, ref = g[name], r[name]
        if got.ndim == 3:   # [B, H, L]: one slice per (b, h)
            got, ref = got[..., None], ref[..., None]
        err = rel_err(got, ref)
        assert err <= tol, f"{name}: {err:.3e}"


@pytest.mark.parametrize("dims", [(128, 128), (64, 64), (64, 128), (128, 64)],
                         ids=lambda d: f"dk{d[0]}dv{d[1]}")
@pytest.mark.parametrize("dt", DTYPES, ids=lambda d: str(d)[6:])
@pytest.mark.parametrize("mode", MODES, ids=lambda m: gi.MODE_NAMES[m])
def test_backward_parity(mode, dt, dims):
    dk, dv = dims
    x = grads_inputs(2, 2, 200, dk, dv, dt, mode, seed=6000 + 10 * mode + dk + dv)
    check(run_bwd(x), oracle_bwd(x), TOL[dt])


@pytest.mark.parametrize("L", [1, 15, 16, 17, 32, 33, 64, 97])
def test_backward_lengths_and_zero_state(L):
    for mode in MODES:
        x = grads_inputs(1, 3, L, 128, 128, torch.bfloat16, mode, seed=6100 + L + mode, s0_std=0.0,
                         final=False)
        check(run_bwd(x), oracle_bwd(x), 2e-2)


@pytest.mark.parametrize("C", [16, 32])
@pytest.mark.parametrize("mode", [gi.ALPHA_SCALAR, gi.ALPHA_CHANNEL], ids=lambda m: gi.MODE_NAMES[m])
def test_backward_chunk_sizes(C, mode):
    x = grads_inputs(1, 2, 150, 128, 128, torch.bfloat16, mode, seed=6200 + C + mode)
    check(run_bwd(x, C), oracle_bwd(x), 2e-2)


# (B, H, L, d_k, d_v, S0): more than 256 chunks of 32 tokens, so every
# gradient workgroup walks a run of 2..4 chunks and carries the state across
# it; with an odd chunk count per head the runs cross into the next head,
# which starts from S0 (or zero), and the head before ends on a ragged chunk
RUNS = [(1, 5, 32 * 60 + 5, 128, 128, True), (2, 4, 32 * 97 + 1, 64, 64, True),
        (1, 9, 32 * 32 + 20, 128, 64, False), (1, 3, 32 * 100, 64, 128, True)]


@pytest.mark.parametrize("case", RUNS, ids=lambda c: f"B{c[0]}H{c[1]}L{c[2]}dk{c[3]}dv{c[4]}s0{int(c[5])}")
@pytest.mark.parametrize("mode", MODES, ids=lambda m: gi.MODE_NAMES[m])
def test_backward_carried_state_runs(case, mode):
    B, H, L, dk, dv, s0 = case
    x = grads_inputs(B, H, L, dk, dv, torch.bfloat16, mode, seed=6270 + L + mode, s0_std=0.1 if s0 else 0.0)
    check(run_bwd(x), oracle_bwd(x), 2e-2)


# (B, H, L, d_k, d_v, dtype, C): the lean path, runs across heads, 16-token
# steps (every chunk's state kept) and fp32
KEEP = [(2, 2, 200, 128, 128, torch.bfloat16, 64), (1, 5, 32 * 60 + 5, 128, 128, torch.bfloat16, 64),
        (1, 3, 97, 64, 128, torch.bfloat16, 16), (1, 2, 150, 64, 64, torch.float32, 64)]


@pytest.mark.parametrize("case", KEEP, ids=lambda c: f"B{c[0]}H{c[1]}L{c[2]}dk{c[3]}dv{c[4]}{str(c[5])[6:]}C{c[6]}")
@pytest.mark.parametrize("mode", MODES, ids=lambda m: gi.MODE_NAMES[m])
def test_kept_forward_and_backward_match(case, mode):
    """A training step through gdr_fwd_chunked_keep and gdr_bwd_chunked_kept
    gives gdr_bwd_chunked's gradients bit for bit, and gdr_fwd_chunked's
    outputs (up to rounding where that call splits a head's scan into
    segments; the keeping forward never does)."""
    B, H, L, dk, dv, dt, C = case
    x = grads_inputs(B, H, L, dk, dv, dt, mode, seed=6700 + L + mode + dk)
    d = {k: (None if t is None else t.cuda()) for k, t in x.items()}
    o, sf, ws = gdr.gdr_fwd_chunked_keep(d["q"], d["k"], d["v"], d["beta"], d["log_alpha"], d["S0"], C)
    o_ref, sf_ref = gdr.gdr_fwd_chunked(d["q"], d["k"], d["v"], d["beta"], d["log_alpha"], d["S0"], C)
    gk = gdr.gdr_bwd_chunked(d["q"], d["k"], d["v"], d["beta"], d["log_alpha"], d["S0"], d["dO"],
                             d["dS_final"], C, workspace=ws, kept=True)
    gr = gdr.gdr_bwd_chunked(d["q"], d["k"], d["v"], d["beta"], d["log_alpha"], d["S0"], d["dO"],
                             d["dS_final"], C)
    torch.cuda.synchronize()
    assert rel_err(o.float().cpu().numpy(), o_ref.float().cpu().numpy()) <= TOL[dt]
    assert rel_err(sf.cpu().numpy(), sf_ref.cpu().numpy()) <= TOL[dt]
    for name in NAMES:
        if gr[name] is None:
            assert gk[name] is None
        else:
            assert torch.equal(gk[name], gr[name]), name


def test_kept_empty_sequence():
    x = grads_inputs(1, 2, 0, 64, 64, torch.bfloat16, gi.ALPHA_SCALAR, seed=6750)
    d = {k: (None if t is None else t.cuda()) for k, t in x.items()}
    o, sf, ws = gdr.gdr_fwd_chunked_keep(d["q"], d["k"], d["v"], d["beta"], d["log_alpha"], d["S0"])
    g = gdr.gdr_bwd_chunked(d["q"], d["k"], d["v"], d["beta"], d["log_alpha"], d["S0"], d["dO"],
                            d["dS_final"], workspace=ws if ws is not None else torch.empty(0, dtype=torch.uint8, device="cuda"),
                            kept=True)
    torch.cuda.synchronize()
    assert torch.equal(sf, d["S0"])
    assert torch.equal(g["dS0"], d["dS_final"])


@pytest.mark.parametrize("dt", DTYPES, ids=lambda d: str(d)[6:])
def test_backward_channel_strong_decay(dt):
    """Channel gates near and past the floor of log alpha at -10: decays of
    e^-80 inside one 8-token span of a chunk, the reference-row scaling at its
    widest; below the floor the gradient of log alpha is zero."""
    x = grads_inputs(1, 2, 96, 128, 128, dt, gi.ALPHA_CHANNEL, seed=6250)
    g = torch.Generator().manual_seed(6251)
    la = -torch.rand(1, 2, 96, 128, generator=g) * 9.5          # in (-9.5, 0]
    la[..., ::7, :] = -9.9                                      # near the floor
    la[..., 5::11, 3::5] = -12.0                                # below it
    x["log_alpha"] = la.contiguous()
    gpu = run_bwd(x)
    floored = x["log_alpha"] < -10.0
    assert np.all(gpu["dlog_alpha"][floored.numpy()] == 0.0)
    ref_x = dict(x, log_alpha=torch.clamp(x["log_alpha"], min=-10.0))
    ref = oracle_bwd(ref_x)
    ref["dlog_alpha"] = np.where(floored.numpy(), 0.0, ref["dlog_alpha"])
    check(gpu, ref, TOL[dt])
    if dt == torch.bfloat16:
        # against the unclamped recurrence: each floored (token, channel)
        # moves the decayed state column by at most e^-10 of its size, and
        # the true gradient of a log alpha below -10 is of that order too
        check(gpu, oracle_bwd(x), TOL[dt])


def test_backward_empty_sequence():
    x = grads_inputs(1, 2, 0, 64, 64, torch.float32, gi.ALPHA_SCALAR, seed=6300)
    g = run_bwd(x)
    assert np.array_equal(g["dS0"], x["dS_final"].numpy())


def test_backward_deterministic():
    x = grads_inputs(2, 2, 300, 128, 128, torch.bfloat16, gi.ALPHA_SCALAR, seed=6400)
    a, b = run_bwd(x), run_bwd(x)
    for name in NAMES:
        assert np.array_equal(a[name], b[name]), name


def test_backward_full_size():
    """The headline shape (B8 H8 L2048 d128, bf16, scalar gates): every
    (b, h) chain against the oracle."""
    x = grads_inputs(8, 8, 2048, 128, 128, torch.bfloat16, gi.ALPHA_SCALAR, seed=6500)
    g = run_bwd(x)
    heads = [(b, h) for b in range(8) for h in range(8)]
    sel = lambda t: None if t is None else torch.stack([t[b, h] for b, h in heads])[None]
    r = oracle.backward(sel(x["q"]), sel(x["k"]), sel(x["v"]), sel(x["beta"]), sel(x["log_alpha"]),
                        sel(x["S0"]), sel(x["dO"]), sel(x["dS_final"]))
    gs = {k: (None if v is None else np.stack([v[b, h] for b, h in heads])[None]) for k, v in g.items()}
    check(gs, r, 2e-2)


def test_backward_full_size_channel():
    """The channel-gate shape (B4 H16 L4096 d128, bf16): every (b, h) chain
    against the oracle."""
    x = grads_inputs(4, 16, 4096, 128, 128, torch.bfloat16, gi.ALPHA_CHANNEL, seed=6600)
    g = run_bwd(x)
    heads = [(b, h) for b in range(4) for h in range(16)]
    sel = lambda t: None if t is None else torch.stack([t[b, h] for b, h in heads])[None]
    r = oracle.backward(sel(x["q"]), sel(x["k"]), sel(x["v"]), sel(x["beta"]), sel(x["log_alpha"]),
                        sel(x["S0"]), sel(x["dO"]), sel(x["dS_final"]))
    gs = {k: (None if v is None else np.stack([v[b, h] for b, h in heads])[None]) for k, v in g.items()}
    check(gs, r, 2e-2)
