"""GPU parity of the packed variable-length forward (gdr_fwd_varlen): every
sequence of the pack against the fp64 oracle run on that sequence alone,
from its own initial state (tolerances as for the fixed-length forward)."""
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
LENGTHS = [1, 31, 32, 33, 64, 100, 0, 257, 5, 63]


def packed(lengths, H, dk, dv, dt, mode, seed, s0_std=0.1, **raw):
    """Inputs for one packed batch: the per-token tensors [H, T, ...] drawn
    as one fixed-length head row of T tokens, S0 [N, H, dv, dk]."""
    T = int(sum(lengths))
    if raw:
        x = gi.raw_inputs((H,), T, dk, dv, dt, mode, seed=seed, **raw)
    else:
        x = gi.chunked_inputs(1, H, T, dk, dv, dt, mode, seed=seed)
        x = {k: (None if v is None else v[0]) for k, v in x.items()}
    g = torch.Generator().manual_seed(seed + 1)
    x["S0"] = torch.randn(len(lengths), H, dv, dk, generator=g) * s0_std if s0_std > 0 else None
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    x["cu"] = torch.from_numpy(cu)
    return x


def run_varlen(x, C=64, pro=0, S_final_is_S0=False):
    d = {k: (None if v is None else v.cuda()) for k, v in x.items()}
    kw = {}
    if S_final_is_S0:
        kw["S_final"] = d["S0"]
    o, S = gdr.gdr_fwd_varlen(d["q"], d["k"], d["v"], d["beta"], d["log_alpha"], d["S0"], d["cu"],
                              C, prologue=pro, **kw)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), S.cpu().numpy()


def oracle_varlen(x, pro=0, heads=None):
    """The oracle on every sequence separately: o [H, T, dv], S [N, H, dv, dk]."""
    cu = x["cu"].numpy()
    N = len(cu) - 1
    H, T = x["q"].shape[:2]
    hs = list(range(H)) if heads is None else heads
    o = np.zeros((len(hs), T, x["v"].shape[-1]))
    S = np.zeros((N, len(hs), x["v"].shape[-1], x["q"].shape[-1]))
    for n in range(N):
        s, e = int(cu[n]), int(cu[n + 1])
        sl = lambda t: None if t is None else t[hs, s:e]
        S0 = None if x["S0"] is None else x["S0"][n][hs]
        if e == s:
            S[n] = 0.0 if S0 is None else S0.double().numpy()
            continue
        on, Sn = oracle.run(sl(x["q"]), sl(x["k"]), sl(x["v"]), sl(x["beta"]), sl(x["log_alpha"]),
                            S0, pro=pro)
        o[:, s:e] = on
        S[n] = Sn
    return o, S


def seq_err(o, S, ro, rS, cu):
    """Max relative error over sequences and heads (each (sequence, head)
    slice scaled by its own reference maximum)."""
    worst = 0.0
    for n in range(len(cu) - 1):
        s, e = int(cu[n]), int(cu[n + 1])
        if e > s:
            worst = max(worst, rel_err(o[None, :, s:e], ro[None, :, s:e]))
        worst = max(worst, rel_err(S[n][None], rS[n][None]))
    return worst


@pytest.mark.parametrize("dt", DTYPES, ids=lambda d: str(d)[6:])
@pytest.mark.parametrize("mode", MODES, ids=lambda m: gi.MODE_NAMES[m])
def test_varlen_parity(mode, dt):
    for dk, dv in ((128, 128), (64, 128)):
        x = packed(LENGTHS, 3, dk, dv, dt, mode, seed=5000 + 10 * mode + dk)
        o, S = run_varlen(x)
        ro, rS = oracle_varlen(x)
        assert seq_err(o, S, ro, rS, x["cu"].numpy()) <= TOL[dt]


@pytest.mark.parametrize("C", [16, 32])
def test_varlen_chunk_sizes_and_zero_state(C):
    for mode in MODES:
        x = packed([40, 17, 0, 96, 3], 2, 128, 64, torch.bfloat16, mode, seed=5100 + C + mode,
                   s0_std=0.0)
        o, S = run_varlen(x, C)
        ro, rS = oracle_varlen(x)
        assert seq_err(o, S, ro, rS, x["cu"].numpy()) <= 2e-2


def test_varlen_equal_lengths_match_the_batched_call_bitwise():
    """B sequences of equal length L packed = the [B, H, L] call: same chunks,
    same kernels, so the same bits."""
    B, H, L = 4, 4, 256
    for mode in MODES:
        y = gi.chunked_inputs(B, H, L, 128, 128, torch.bfloat16, mode, seed=5200 + mode, s0_std=0.1)
        d = {k: (None if v is None else v.cuda()) for k, v in y.items()}
        ob, Sb = gdr.gdr_fwd_chunked(d["q"], d["k"], d["v"], d["beta"], d["log_alpha"], d["S0"], 64)
        pack = lambda t: None if t is None else t.transpose(0, 1).reshape((H, B * L) + t.shape[3:]).contiguous()
        cu = torch.arange(0, B * L + 1, L, dtype=torch.int32, device="cuda")
        ov, Sv = gdr.gdr_fwd_varlen(pack(d["q"]), pack(d["k"]), pack(d["v"]), pack(d["beta"]),
                                    pack(d["log_alpha"]), d["S0"], cu, 64)
        torch.cuda.synchronize()
        assert torch.equal(pack(ob), ov)
        assert torch.equal(Sb, Sv)


def test_varlen_prologue():
    for mode in MODES:
        for dt in DTYPES:
            x = packed(LENGTHS, 2, 128, 128, dt, mode, seed=5300 + mode, raw_qk=True,
                       raw_gates=True)
            o, S = run_varlen(x, pro=3)
            ro, rS = oracle_varlen(x, pro=3)
            assert seq_err(o, S, ro, rS, x["cu"].numpy()) <= TOL[dt]


def test_varlen_in_place_state_and_empty_pack():
    x = packed([50, 0, 70], 2, 64, 64, torch.float32, gi.ALPHA_SCALAR, seed=5400)
    o, S = run_varlen(x, S_final_is_S0=True)
    ro, rS = oracle_varlen(x)
    assert seq_err(o, S, ro, rS, x["cu"].numpy()) <= 1e-4
    assert np.array_equal(S[1], x["S0"][1].numpy())          # empty sequence keeps its state
    # no tokens at all: every final state is its initial state
    y = packed([0, 0, 0], 2, 64, 64, torch.float32, gi.ALPHA_SCALAR, seed=5401)
    _, S = run_varlen(y)
    assert np.array_equal(S, y["S0"].numpy())


def test_varlen_many_sequences_sampled():
    """64 sequences with lengths from 1 to 1000 tokens (T about 32 K per head),
    8 heads; the oracle checks four heads of every sequence."""
    rng = np.random.default_rng(55)
    lengths = rng.integers(1, 1000, size=64)
    lengths[[3, 17]] = [2048, 1]
    x = packed(list(lengths), 8, 128, 128, torch.bfloat16, gi.ALPHA_SCALAR, seed=5500)
    o, S = run_varlen(x)
    heads = [0, 2, 5, 7]
    ro, rS = oracle_varlen(x, heads=heads)
    assert seq_err(o[heads], S[:, heads], ro, rS, x["cu"].numpy()) <= 2e-2


def test_varlen_more_sequences_than_one_planning_tile():
    """1500 short sequences (the per-sequence plan runs in tiles of 1024),
    including empty ones."""
    rng = np.random.default_rng(56)
    lengths = rng.integers(0, 40, size=1500)
    x = packed(list(lengths), 2, 64, 64, torch.float32, gi.ALPHA_SCALAR, seed=5600)
    o, S = run_varlen(x)
    ro, rS = oracle_varlen(x)
    assert seq_err(o, S, ro, rS, x["cu"].numpy()) <= 1e-4
