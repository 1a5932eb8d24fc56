"""Why Gated DeltaNet-2 is not built: the pages do not force one update.

"Linear Attention Architectures: Mechanisms, Trade-offs, and Cross-Layer
Routing", Sec. 3 (the Gated DeltaNet-2 paragraph and Eq. (13)) keeps only
prose about the update, whose formulas are lost from the text: a
channel-wise erase gate e acts on the key side, a channel-wise write gate w
on the value side, the decay is Kimi's channel-wise one, and the update
reduces to Kimi Delta Attention when both gates collapse to the scalar beta,
and further to Gated DeltaNet when the decay is scalar too.

Two natural updates satisfy every one of those statements (W d_v x d_k,
Wbar = W Diag(alpha), kappa the key):
  R1  W = Wbar + (w . v - Wbar (e . kappa)) kappa^T      erase gate inside the prediction
  R2  W = Wbar - (Wbar kappa) (e . kappa)^T + (w . v) kappa^T
                                                        erase gate on the row side of the projector
These tests check both reductions for both readings against the fp64 oracle,
and that the two readings disagree for general gates: the pages leave the
choice open, so no oracle (and no kernel) is written for either.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle


def _run(reading, q, k, v, la, e, w):
    """Token loop of a candidate update; arrays [L, d] (la: [L, dk])."""
    L, dk = k.shape
    dv = v.shape[1]
    W = np.zeros((dv, dk))
    out = np.zeros((L, dv))
    for t in range(L):
        Wb = W * np.exp(la[t])[None, :]
        kap = k[t]
        if reading == 1:
            W = Wb + np.outer(w[t] * v[t] - Wb @ (e[t] * kap), kap)
        else:
            W = Wb - np.outer(Wb @ kap, e[t] * kap) + np.outer(w[t] * v[t], kap)
        out[t] = W @ q[t]
    return out, W


def _inputs(L=24, dk=8, dv=6, seed=0):
    rng = np.random.default_rng(seed)
    unit = lambda x: x / np.linalg.norm(x, axis=-1, keepdims=True)
    q = unit(rng.standard_normal((L, dk)))
    k = unit(rng.standard_normal((L, dk)))
    v = rng.standard_normal((L, dv))
    beta = 1 / (1 + np.exp(-rng.standard_normal(L)))
    la = -np.log1p(np.exp(rng.standard_normal((L, dk)) + 1.0))
    return q, k, v, beta, la


def _oracle(q, k, v, beta, la):
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a))[None, None]
    o, S = oracle.run(t(q), t(k), t(v), t(beta), t(la), None)
    return o[0, 0], S[0, 0]


def test_both_readings_reduce_to_kimi_delta_attention():
    q, k, v, beta, la = _inputs()
    ref_o, ref_S = _oracle(q, k, v, beta, la)          # channel-wise decay
    e = np.repeat(beta[:, None], k.shape[1], axis=1)
    w = np.repeat(beta[:, None], v.shape[1], axis=1)
    for r in (1, 2):
        o, S = _run(r, q, k, v, la, e, w)
        assert np.abs(o - ref_o).max() < 1e-12 and np.abs(S - ref_S).max() < 1e-12


def test_both_readings_reduce_to_gated_deltanet():
    q, k, v, beta, la = _inputs(seed=1)
    las = np.repeat(la[:, :1], k.shape[1], axis=1)     # one decay per token
    ref_o, ref_S = _oracle(q, k, v, beta, las[:, 0])   # scalar gates
    e = np.repeat(beta[:, None], k.shape[1], axis=1)
    w = np.repeat(beta[:, None], v.shape[1], axis=1)
    for r in (1, 2):
        o, S = _run(r, q, k, v, las, e, w)
        assert np.abs(o - ref_o).max() < 1e-12 and np.abs(S - ref_S).max() < 1e-12


def test_the_readings_disagree_for_channel_wise_gates():
    q, k, v, beta, la = _inputs(seed=2)
    rng = np.random.default_rng(3)
    e = 1 / (1 + np.exp(-rng.standard_normal((len(beta), k.shape[1]))))
    w = 1 / (1 + np.exp(-rng.standard_normal((len(beta), v.shape[1]))))
    o1, S1 = _run(1, q, k, v, la, e, w)
    o2, S2 = _run(2, q, k, v, la, e, w)
    rel = np.abs(o1 - o2).max() / np.abs(o1).max()
    assert rel > 1e-2, rel
