"""fp64 CPU oracle for the gated delta-rule memory (ctypes wrapper).

TEST INFRASTRUCTURE ONLY: only ``tests/``, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import this package.  The product
path (``gated_delta_rule_88_amd``) never imports, links or executes it, and
this package imports nothing from the product path.

The arithmetic lives in ``gdr_oracle.c`` (plain C, double precision, one
token at a time); see that file's header for the recurrence and the passages
it follows.  This wrapper only converts arrays to contiguous float64 and
calls it.
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


def max_threads() -> int:
    return int(_load().gdr_oracle_max_threads())


def run(q, k, v, beta, log_alpha=None, S0=None, mode: int | None = None,
        no_delta: bool = False, nthreads: int = 0):
    """Token-by-token fp64 recurrence.

    q, k: [..., L, dk]; v: [..., L, dv]; beta: [..., L];
    log_alpha: None | [..., L] | [..., L, dk]; S0: None | [..., dv, dk].
    The leading dimensions (batch, head, ...) are independent chains.
    Returns (o [..., L, dv], S_final [..., dv, dk]) as float64 arrays.
    """
    q, k, v, beta = _f64(q), _f64(k), _f64(v), _f64(beta)
    la, s0 = _f64(log_alpha), _f64(S0)
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
