"""Shared helpers for the GPU parity tests."""
from __future__ import annotations

import numpy as np
import torch

import gated_delta_rule_88_amd as gdr
import gdr_inputs as gi
import oracle

# Tolerances stated for the method: max relative error (per (batch, head)
# slice: max |x - ref| / max |ref|, then the max over slices), against the
# fp64 oracle run on the same rounded inputs.
TOL = {torch.float32: 1e-4, torch.bfloat16: 2e-2}


def rel_err(x, ref) -> float:
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if ref.size == 0:
        return 0.0
    lead = ref.shape[:2]
    xs = x.reshape(lead + (-1,))
    rs = ref.reshape(lead + (-1,))
    num = np.abs(xs - rs).max(axis=-1)
    den = np.maximum(np.abs(rs).max(axis=-1), 1e-30)
    return float((num / den).max())


def to_dev(d: dict, dev="cuda") -> dict:
    return {k: (None if v is None else v.to(dev)) for k, v in d.items()}


def run_chunked(x: dict, C: int = 64, S_final_is_S0: bool = False):
    d = to_dev(x)
    kw = {}
    if S_final_is_S0 and d["S0"] is not None:
        kw["S_final"] = d["S0"]
    o, S = gdr.gdr_fwd_chunked(d["q"], d["k"], d["v"], d["beta"], d["log_alpha"], d["S0"], C,
                               **kw)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), S.cpu().numpy()


def oracle_chunked(x: dict, heads=None):
    """Oracle on all (b, h) chains, or on the listed (b, h) pairs."""
    if heads is None:
        return oracle.run(x["q"], x["k"], x["v"], x["beta"], x["log_alpha"], x["S0"])
    sel = lambda t: None if t is None else torch.stack([t[b, h] for b, h in heads])[None]
    o, S = oracle.run(sel(x["q"]), sel(x["k"]), sel(x["v"]), sel(x["beta"]), sel(x["log_alpha"]),
                      sel(x["S0"]))
    return o[0], S[0]


def pick(arr, heads):
    return np.stack([arr[b, h] for b, h in heads])[None]
