"""The chunked forward without a workspace argument (gdr_fwd_chunked_noalloc)
against gdr_fwd_chunked through the C ABI: two calls in a row on the same
GPU, the second smaller than the first, each equal to the plain entry
point's result (same kernels, so bit for bit) and within the bf16 / fp32
tolerance of the fp64 oracle."""
from __future__ import annotations

import pytest
import torch

import gated_delta_rule_88_amd as gdr
import gdr_inputs as gi
from gpu_common import TOL, oracle_chunked, rel_err, to_dev

pytestmark = pytest.mark.gpu


def _both(x, C):
    d = to_dev(x)
    ref_o, ref_S = gdr.gdr_fwd_chunked(d["q"], d["k"], d["v"], d["beta"], d["log_alpha"], d["S0"], C)
    o = torch.full_like(ref_o, float("nan"))
    S = torch.full_like(ref_S, float("nan"))
    gdr.gdr_fwd_chunked_noalloc(d["q"], d["k"], d["v"], d["beta"], d["log_alpha"], d["S0"], C,
                                o=o, S_final=S)
    torch.cuda.synchronize()
    return (o, S), (ref_o, ref_S)


def test_noalloc_two_calls_second_smaller():
    # first: the Gated DeltaNet workload at full size (about 19 MB of scratch)
    w = gi.GDN_BF16
    big = gi.chunked_inputs(w.B, w.H, w.L, w.dk, w.dv, w.dtype, w.mode, seed=8800, s0_std=0.1)
    (o, S), (ro, rS) = _both(big, w.C)
    assert torch.equal(o, ro) and torch.equal(S, rS)
    # second: smaller, with a ragged last chunk; the array still holds the
    # first call's records
    small = gi.chunked_inputs(2, 3, 200, 128, 64, torch.bfloat16, gi.ALPHA_CHANNEL, seed=8801,
                              s0_std=0.1)
    (o, S), (ro, rS) = _both(small, 64)
    assert torch.equal(o, ro) and torch.equal(S, rS)
    eo, eS = oracle_chunked(small)
    assert rel_err(o.float().cpu().numpy(), eo) <= TOL[torch.bfloat16]
    assert rel_err(S.cpu().numpy(), eS) <= TOL[torch.bfloat16]


@pytest.mark.parametrize("mode", [gi.ALPHA_NONE, gi.ALPHA_SCALAR, gi.ALPHA_CHANNEL],
                         ids=lambda m: gi.MODE_NAMES[m])
def test_noalloc_modes_fp32(mode):
    x = gi.chunked_inputs(1, 2, 100, 64, 64, torch.float32, mode, seed=8810 + mode, s0_std=0.1)
    (o, S), (ro, rS) = _both(x, 32)
    assert torch.equal(o, ro) and torch.equal(S, rS)
    eo, eS = oracle_chunked(x)
    assert rel_err(o.cpu().numpy(), eo) <= TOL[torch.float32]
    assert rel_err(S.cpu().numpy(), eS) <= TOL[torch.float32]


def test_noalloc_refuses_a_call_beyond_the_scratch():
    q = torch.zeros(8, 8, 65536, 128, dtype=torch.bfloat16, device="cuda")
    beta = torch.zeros(8, 8, 65536, device="cuda")
    la = torch.zeros(8, 8, 65536, 128, device="cuda")
    with pytest.raises(gdr.GdrError) as e:
        gdr.gdr_fwd_chunked_noalloc(q, q, q, beta, la, None, 64)
    assert e.value.status == gdr.GDR_ERR_SCRATCH_TOO_SMALL


def test_noalloc_empty_and_zero_length():
    x = gi.chunked_inputs(2, 3, 0, 64, 128, torch.bfloat16, gi.ALPHA_SCALAR, seed=8820,
                          s0_std=0.5)
    d = to_dev(x)
    o, S = gdr.gdr_fwd_chunked_noalloc(d["q"], d["k"], d["v"], d["beta"], d["log_alpha"], d["S0"])
    torch.cuda.synchronize()
    assert torch.equal(S.cpu(), x["S0"]) and o.numel() == 0
