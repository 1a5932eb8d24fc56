"""fp64 CPU oracle for the gated delta-rule memory (ctypes wrapper).

TEST INFRASTRUCTURE ONLY: only ``tests/``, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import this package.  The product
path (``gated_delta_rule_88_amd``) never imports, links or executes it, and
this package imports nothing from the product path.

The recurrence and its reverse mode (gradients, for training) live in
``gdr_oracle.c`` (plain C, double precision, one token at a time); see that
file for the recurrence, the passages it follows and the per-token chain
rule of the backward.  This wrapper converts arrays to contiguous float64 and calls
it.  The only arithmetic written here is the optional input-side prologue
(``prologue``): unit-norm queries and keys and the sigmoid gates, applied
elementwise in float64 before the recurrence runs.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdr_oracle.c")
LIB_PATH = os.path.join(_HERE, "libgdr_oracle.so")

ALPHA_NONE, ALPHA_SCALAR, ALPHA_CHANNEL = 0, 1, 2
PRO_L2NORM_QK, PRO_GATES = 1, 2
NORM_EPS = 1e-6

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (OpenMP, strict IEEE double arithmetic)."""
    if not force and os.path.exists(LIB_PATH):
        return LIB_PATH
    tmp = LIB_PATH + ".tmp"
    cmd = ["gcc", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp", "-fPIC",
           "-shared", "-std=c99", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        lib = ctypes.CDLL(LIB_PATH)
        dp = ctypes.POINTER(ctypes.c_double)
        lib.gdr_oracle_run.argtypes = [ctypes.c_int] * 6 + [dp] * 8 + [ctypes.c_int]
        lib.gdr_oracle_run.restype = ctypes.c_int
        lib.gdr_oracle_max_threads.restype = ctypes.c_int
        lib.gdr_oracle_backward.argtypes = [ctypes.c_int] * 5 + [dp] * 14 + [ctypes.c_int]
        lib.gdr_oracle_backward.restype = ctypes.c_int
        _lib = lib
    return _lib


def _f64(x):
    if x is None:
        return None
    if hasattr(x, "detach"):  # torch tensor: upcast exactly (bf16/fp32 -> fp64)
        x = x.detach().to("cpu").double().numpy()
    return np.ascontiguousarray(x, dtype=np.float64)


def _ptr(a):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def l2_normalise(x):
    """x / max(||x||_2, 1e-6) along the last axis, in float64.

    Keys (and queries) of unit length are what make a read by a stored key
    return its value exactly when the keys are orthogonal ("linear attention
    and its gated descendants", section "DeltaNet"); the floor keeps an
    all-zero vector at zero instead of dividing by zero.
    """
    x = _f64(x)
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
    return x / np.maximum(n, NORM_EPS)


def sigmoid(x):
    """1 / (1 + exp(-x)) in float64, evaluated as exp(-|x|) ratios so that
    neither tail overflows (the write-strength and decay gates of the
    minimal pseudocode in "Linear Attention & DeltaNet" are sigmoids)."""
    x = _f64(x)
    e = np.exp(-np.abs(x))
    return np.where(x >= 0, 1.0 / (1.0 + e), e / (1.0 + e))


def log_sigmoid(x):
    """log(sigmoid(x)) = min(x, 0) - log(1 + exp(-|x|)) in float64: the log
    of a sigmoid decay gate, finite for every finite x."""
    x = _f64(x)
    return np.minimum(x, 0.0) - np.log1p(np.exp(-np.abs(x)))


def prologue(q, k, beta, log_alpha, flags: int):
    """The input-side steps a caller may ask the library to apply.

    flags & PRO_L2NORM_QK: q and k are divided by their L2 norms.
    flags & PRO_GATES: beta and log_alpha hold raw pre-activations b, a; the
    gates are beta = sigmoid(b) and alpha = sigmoid(a), so log alpha =
    log_sigmoid(a).  Returns float64 (q, k, beta, log_alpha); absent
    log_alpha stays None.
    """
    q, k, beta, la = _f64(q), _f64(k), _f64(beta), _f64(log_alpha)
    if flags & ~(PRO_L2NORM_QK | PRO_GATES):
        raise ValueError(f"unknown prologue bits {flags}")
    if flags & PRO_L2NORM_QK:
        q, k = l2_normalise(q), l2_normalise(k)
    if flags & PRO_GATES:
        beta = sigmoid(beta)
        la = None if la is None else log_sigmoid(la)
    return q, k, beta, la


def max_threads() -> int:
    return int(_load().gdr_oracle_max_threads())


def run(q, k, v, beta, log_alpha=None, S0=None, mode: int | None = None,
        no_delta: bool = False, nthreads: int = 0, pro: int = 0):
    """Token-by-token fp64 recurrence.

    q, k: [..., L, dk]; v: [..., L, dv]; beta: [..., L];
    log_alpha: None | [..., L] | [..., L, dk]; S0: None | [..., dv, dk].
    The leading dimensions (batch, head, ...) are independent chains.
    ``pro`` applies ``prologue`` to q, k, beta and log_alpha first.
    Returns (o [..., L, dv], S_final [..., dv, dk]) as float64 arrays.
    """
    q, k, v, beta = _f64(q), _f64(k), _f64(v), _f64(beta)
    la, s0 = _f64(log_alpha), _f64(S0)
    if pro:
        q, k, beta, la = prologue(q, k, beta, la, pro)
    lead = q.shape[:-2]
    L, dk = q.shape[-2:]
    dv = v.shape[-1]
    if mode is None:
        mode = ALPHA_NONE if la is None else (ALPHA_CHANNEL if la.shape == q.shape
                                              else ALPHA_SCALAR)
    if mode == ALPHA_NONE:
        la = None
    if k.shape != q.shape or v.shape[:-1] != q.shape[:-1] or beta.shape != q.shape[:-1]:
        raise ValueError("shape mismatch among q, k, v, beta")
    if mode == ALPHA_SCALAR and (la is None or la.shape != beta.shape):
        raise ValueError("scalar log_alpha must have the shape of beta")
    if mode == ALPHA_CHANNEL and (la is None or la.shape != q.shape):
        raise ValueError("channel log_alpha must have the shape of q")
    if s0 is not None and s0.shape != lead + (dv, dk):
        raise ValueError("S0 must be [..., dv, dk]")
    BH = int(np.prod(lead)) if lead else 1
    o = np.zeros(lead + (L, dv), dtype=np.float64)
    S = np.zeros(lead + (dv, dk), dtype=np.float64)
    rc = _load().gdr_oracle_run(BH, L, dk, dv, int(mode), int(bool(no_delta)),
                                _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(la), _ptr(s0),
                                _ptr(o), _ptr(S), int(nthreads))
    if rc != 0:
        raise RuntimeError("oracle run failed")
    return o, S


def backward(q, k, v, beta, log_alpha=None, S0=None, do=None, dS_final=None,
             mode: int | None = None, nthreads: int = 0, pro: int = 0):
    """Gradients of the token recurrence (reverse mode, fp64), for a loss
    whose gradient with respect to the outputs is ``do`` [..., L, dv] and
    with respect to the final state ``dS_final`` (None = 0).

    Shapes as ``run``.  Returns a dict with dq, dk [..., L, dk], dv
    [..., L, dv], dbeta [..., L], dlog_alpha (None | like log_alpha) and dS0
    [..., dv, dk].  With ``pro`` the inputs are taken raw, the prologue is
    applied first and the gradients are with respect to the raw inputs
    (chained through the prologue by ``prologue_backward``).
    """
    if pro:
        raw = (q, k, beta, log_alpha)
        q, k, beta, log_alpha = prologue(q, k, beta, log_alpha, pro)
    q, k, v, beta = _f64(q), _f64(k), _f64(v), _f64(beta)
    la, s0, dout, dsf = _f64(log_alpha), _f64(S0), _f64(do), _f64(dS_final)
    lead = q.shape[:-2]
    L, dk = q.shape[-2:]
    dv = v.shape[-1]
    if mode is None:
        mode = ALPHA_NONE if la is None else (ALPHA_CHANNEL if la.shape == q.shape
                                              else ALPHA_SCALAR)
    if mode == ALPHA_NONE:
        la = None
    if dout is None or dout.shape != v.shape:
        raise ValueError("do must have the shape of v")
    if dsf is not None and dsf.shape != lead + (dv, dk):
        raise ValueError("dS_final must be [..., dv, dk]")
    BH = int(np.prod(lead)) if lead else 1
    g = dict(dq=np.zeros(q.shape), dk=np.zeros(q.shape), dv=np.zeros(v.shape),
             dbeta=np.zeros(beta.shape), dlog_alpha=None if la is None else np.zeros(la.shape),
             dS0=np.zeros(lead + (dv, dk)))
    rc = _load().gdr_oracle_backward(BH, L, dk, dv, int(mode), _ptr(q), _ptr(k), _ptr(v),
                                     _ptr(beta), _ptr(la), _ptr(s0), _ptr(dout), _ptr(dsf),
                                     _ptr(g["dq"]), _ptr(g["dk"]), _ptr(g["dv"]),
                                     _ptr(g["dbeta"]), _ptr(g["dlog_alpha"]), _ptr(g["dS0"]),
                                     int(nthreads))
    if rc != 0:
        raise RuntimeError("oracle backward failed")
    if pro:
        g = prologue_backward(*raw, g, pro)
    return g


def prologue_backward(q_raw, k_raw, beta_raw, la_raw, g: dict, flags: int) -> dict:
    """Chain gradients with respect to the prologue's outputs back to its raw
    inputs: for y = x / max(||x||, eps), dx = (dy - y (y . dy)) / ||x|| while
    ||x|| > eps (dx = dy / eps below the floor); for beta = sigmoid(b),
    db = dbeta beta (1 - beta); for log alpha = log sigmoid(a),
    da = dlog_alpha (1 - sigmoid(a))."""
    g = dict(g)
    if flags & PRO_L2NORM_QK:
        for name, x in (("dq", q_raw), ("dk", k_raw)):
            x = _f64(x)
            n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
            y = x / np.maximum(n, NORM_EPS)
            dy = g[name]
            inside = n > NORM_EPS
            g[name] = np.where(inside, (dy - y * np.sum(y * dy, axis=-1, keepdims=True))
                               / np.maximum(n, NORM_EPS), dy / NORM_EPS)
    if flags & PRO_GATES:
        b = sigmoid(beta_raw)
        g["dbeta"] = g["dbeta"] * b * (1.0 - b)
        if g["dlog_alpha"] is not None:
            g["dlog_alpha"] = g["dlog_alpha"] * (1.0 - sigmoid(la_raw))
    return g
