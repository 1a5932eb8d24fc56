"""Gated delta-rule memory for MI355X: Python binding over libgdr.so.

The binding only marshals arguments: it checks devices, dtypes, shapes and
contiguity of torch tensors, allocates outputs (and the chunked forward's
workspace) with torch, and passes raw device pointers plus the current HIP
stream to the C ABI declared in ``include/gdr.h``.  Every step of the
computation runs in the library's HIP kernels.  There is no fallback: if
``libgdr.so`` is missing or cannot be loaded, importing a function raises.

Functions carry the C names:

* ``gdr_fwd_chunked(q, k, v, beta, log_alpha=None, S0=None, chunk=64, ...)``
  -> ``(o, S_final)``: chunkwise forward over ``[B, H, L, d]`` inputs.
* ``gdr_decode_step(q, k, v, beta, log_alpha, S, o=None)`` -> ``o``: one
  recurrent step over ``[N, H, d]`` inputs, updating ``S`` in place.
* ``gdr_fwd_chunked_workspace_size``, ``gdr_abi_version``,
  ``gdr_status_string``.
"""
from __future__ import annotations

import ctypes
import functools
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libgdr.so")

GDR_OK, GDR_ERR_INVALID_ARG, GDR_ERR_UNSUPPORTED = 0, 1, 2
GDR_ERR_WORKSPACE_TOO_SMALL, GDR_ERR_HIP, GDR_ERR_SCRATCH_TOO_SMALL = 3, 4, 5
GDR_NOALLOC_SCRATCH_BYTES = 64 << 20
GDR_F32, GDR_BF16 = 0, 1
GDR_ALPHA_NONE, GDR_ALPHA_SCALAR, GDR_ALPHA_CHANNEL = 0, 1, 2
GDR_PRO_L2NORM_QK, GDR_PRO_GATES = 1, 2

_SIZE_MAX = ctypes.c_size_t(-1).value

EXPORTED = ("gdr_abi_version", "gdr_status_string", "gdr_fwd_chunked_workspace_size",
            "gdr_fwd_chunked_token_step",
            "gdr_fwd_chunked", "gdr_fwd_chunked_ex", "gdr_fwd_chunked_noalloc", "gdr_fwd_varlen_workspace_size",
            "gdr_fwd_varlen", "gdr_bwd_chunked_workspace_size", "gdr_bwd_chunked",
            "gdr_fwd_chunked_keep", "gdr_bwd_chunked_kept",
            "gdr_decode_step", "gdr_decode_step_ex")

_lib = None


class GdrError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {gdr_status_string(status)} (status {status})")
        self.status = status


def load_library():
    """Load libgdr.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m gated_delta_rule_88_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, sz, i = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
    lib.gdr_abi_version.restype = i
    lib.gdr_status_string.argtypes = [i]
    lib.gdr_status_string.restype = ctypes.c_char_p
    lib.gdr_fwd_chunked_workspace_size.argtypes = [i] * 8
    lib.gdr_fwd_chunked_workspace_size.restype = sz
    lib.gdr_fwd_chunked_token_step.argtypes = [i] * 3
    lib.gdr_fwd_chunked_token_step.restype = i
    lib.gdr_fwd_chunked.argtypes = [i] * 7 + [vp] * 4 + [i] + [vp] * 5 + [sz, vp]
    lib.gdr_fwd_chunked.restype = i
    lib.gdr_fwd_chunked_ex.argtypes = lib.gdr_fwd_chunked.argtypes + [ctypes.c_uint]
    lib.gdr_fwd_chunked_ex.restype = i
    lib.gdr_fwd_chunked_noalloc.argtypes = [i] * 7 + [vp] * 4 + [i] + [vp] * 5
    lib.gdr_fwd_chunked_noalloc.restype = i
    lib.gdr_fwd_varlen_workspace_size.argtypes = [i] * 8
    lib.gdr_fwd_varlen_workspace_size.restype = sz
    lib.gdr_fwd_varlen.argtypes = [i] * 3 + [vp] + [i] * 4 + [vp] * 4 + [i] + [vp] * 5 + [sz, vp,
                                                                                        ctypes.c_uint]
    lib.gdr_fwd_varlen.restype = i
    lib.gdr_bwd_chunked_workspace_size.argtypes = [i] * 8
    lib.gdr_bwd_chunked_workspace_size.restype = sz
    lib.gdr_bwd_chunked.argtypes = [i] * 7 + [vp] * 4 + [i] + [vp] * 11 + [sz, vp]
    lib.gdr_bwd_chunked.restype = i
    lib.gdr_bwd_chunked_kept.argtypes = lib.gdr_bwd_chunked.argtypes
    lib.gdr_bwd_chunked_kept.restype = i
    lib.gdr_fwd_chunked_keep.argtypes = lib.gdr_fwd_chunked.argtypes
    lib.gdr_fwd_chunked_keep.restype = i
    lib.gdr_decode_step.argtypes = [i] * 5 + [vp] * 4 + [i] + [vp] * 4
    lib.gdr_decode_step.restype = i
    lib.gdr_decode_step_ex.argtypes = lib.gdr_decode_step.argtypes + [ctypes.c_uint]
    lib.gdr_decode_step_ex.restype = i
    _lib = lib
    return lib


def gdr_abi_version() -> int:
    return int(load_library().gdr_abi_version())


def gdr_status_string(status: int) -> str:
    return load_library().gdr_status_string(int(status)).decode()


def gdr_fwd_chunked_token_step(C: int, dtype: int, alpha_mode: int) -> int:
    """Tokens per state step the chunked forward executes for chunk length C
    (0 for arguments outside the domain)."""
    return int(load_library().gdr_fwd_chunked_token_step(int(C), int(dtype), int(alpha_mode)))


def _dtype_code(t: torch.dtype) -> int:
    if t == torch.bfloat16:
        return GDR_BF16
    if t == torch.float32:
        return GDR_F32
    raise TypeError(f"q/k/v must be bfloat16 or float32, got {t}")


def _mode_of(log_alpha, q) -> int:
    if log_alpha is None:
        return GDR_ALPHA_NONE
    return GDR_ALPHA_CHANNEL if log_alpha.dim() == q.dim() else GDR_ALPHA_SCALAR


def _ptr(t):
    # a plain int: the c_void_p argtype converts it without a Python object per call
    return None if t is None else t.data_ptr()


def _check(t, name, dtype, device, shape):
    if t is None:
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    td = t.device
    if td.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor, got {td}")
    if td != device:
        raise ValueError(f"{name} is on {td}, expected {device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.shape != shape:
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


@functools.lru_cache(maxsize=256)
def _chunked_ws(B, H, L, dk, dv, C, code, mode) -> int:
    return int(load_library().gdr_fwd_chunked_workspace_size(B, H, L, dk, dv, C, code, mode))


def gdr_fwd_chunked_workspace_size(B, H, L, d_k, d_v, C, dtype, alpha_mode) -> int:
    return int(load_library().gdr_fwd_chunked_workspace_size(B, H, L, d_k, d_v, C, dtype,
                                                             alpha_mode))


def _prepare_fwd_chunked(q, k, v, beta, log_alpha, S0, chunk, o, S_final, write_final, workspace,
                         stream, prologue):
    """Checks and allocations of a gdr_fwd_chunked call; returns the C
    function, its arguments, its name and (o, S_final)."""
    lib = load_library()
    if q.dim() != 4:
        raise ValueError("q must be [B, H, L, d_k]")
    B, H, L, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    dt = q.dtype
    code = _dtype_code(dt)
    mode = _mode_of(log_alpha, q)
    _check(q, "q", dt, dev, (B, H, L, dk))
    _check(k, "k", dt, dev, (B, H, L, dk))
    _check(v, "v", dt, dev, (B, H, L, dv))
    _check(beta, "beta", torch.float32, dev, (B, H, L))
    if mode == GDR_ALPHA_SCALAR:
        _check(log_alpha, "log_alpha", torch.float32, dev, (B, H, L))
    elif mode == GDR_ALPHA_CHANNEL:
        _check(log_alpha, "log_alpha", torch.float32, dev, (B, H, L, dk))
    _check(S0, "S0", torch.float32, dev, (B, H, dv, dk))
    if o is None:
        o = torch.empty((B, H, L, dv), dtype=dt, device=dev)
    _check(o, "o", dt, dev, (B, H, L, dv))
    if S_final is None and write_final:
        S_final = torch.empty((B, H, dv, dk), dtype=torch.float32, device=dev)
    _check(S_final, "S_final", torch.float32, dev, (B, H, dv, dk))
    need = _chunked_ws(B, H, L, dk, dv, chunk, code, mode)
    if need == _SIZE_MAX:
        raise GdrError(GDR_ERR_UNSUPPORTED, "gdr_fwd_chunked_workspace_size")
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    args = (B, H, L, dk, dv, chunk, code, _ptr(q), _ptr(k), _ptr(v), _ptr(beta), mode,
            _ptr(log_alpha), _ptr(S0), _ptr(o), _ptr(S_final), _ptr(workspace), ws_bytes,
            _stream(stream))
    if prologue:
        return lib.gdr_fwd_chunked_ex, args + (int(prologue),), "gdr_fwd_chunked_ex", (o, S_final), workspace
    return lib.gdr_fwd_chunked, args, "gdr_fwd_chunked", (o, S_final), workspace


def gdr_fwd_chunked(q, k, v, beta, log_alpha=None, S0=None, chunk: int = 64, *,
                    o=None, S_final=None, write_final: bool = True, workspace=None,
                    stream=None, prologue: int = 0):
    """Chunkwise forward.  q, k [B,H,L,dk]; v [B,H,L,dv] (bf16 or fp32);
    beta [B,H,L] fp32; log_alpha None | [B,H,L] | [B,H,L,dk] fp32;
    S0 None | [B,H,dv,dk] fp32.  Returns (o, S_final or None).
    Pass S_final=S0 to update the state in place.  ``prologue`` (a set of
    GDR_PRO_* bits) asks the library to L2-normalise q and k and/or to take
    beta and log_alpha as raw gate pre-activations (gdr_fwd_chunked_ex)."""
    fn, args, name, out, _ = _prepare_fwd_chunked(q, k, v, beta, log_alpha, S0, chunk, o, S_final,
                                                  write_final, workspace, stream, prologue)
    st = fn(*args)
    if st != GDR_OK:
        raise GdrError(st, name)
    return out


def gdr_fwd_chunked_noalloc(q, k, v, beta, log_alpha=None, S0=None, chunk: int = 64, *,
                            o=None, S_final=None, write_final: bool = True, stream=None):
    """gdr_fwd_chunked without a workspace: the library's fixed per-device
    scratch array (GDR_NOALLOC_SCRATCH_BYTES) serves instead, so the C call
    allocates nothing.  Pass ``o`` (and ``S_final``) to keep the whole call
    free of allocations; otherwise they are allocated here, as in
    gdr_fwd_chunked.  Calls that overlap on one GPU race on the shared
    array."""
    lib = load_library()
    if q.dim() != 4:
        raise ValueError("q must be [B, H, L, d_k]")
    B, H, L, dk = q.shape
    dv = v.shape[-1]
    dev, dt = q.device, q.dtype
    code = _dtype_code(dt)
    mode = _mode_of(log_alpha, q)
    _check(q, "q", dt, dev, (B, H, L, dk))
    _check(k, "k", dt, dev, (B, H, L, dk))
    _check(v, "v", dt, dev, (B, H, L, dv))
    _check(beta, "beta", torch.float32, dev, (B, H, L))
    if mode == GDR_ALPHA_SCALAR:
        _check(log_alpha, "log_alpha", torch.float32, dev, (B, H, L))
    elif mode == GDR_ALPHA_CHANNEL:
        _check(log_alpha, "log_alpha", torch.float32, dev, (B, H, L, dk))
    _check(S0, "S0", torch.float32, dev, (B, H, dv, dk))
    if o is None:
        o = torch.empty((B, H, L, dv), dtype=dt, device=dev)
    _check(o, "o", dt, dev, (B, H, L, dv))
    if S_final is None and write_final:
        S_final = torch.empty((B, H, dv, dk), dtype=torch.float32, device=dev)
    _check(S_final, "S_final", torch.float32, dev, (B, H, dv, dk))
    st = lib.gdr_fwd_chunked_noalloc(B, H, L, dk, dv, chunk, code, _ptr(q), _ptr(k), _ptr(v),
                                     _ptr(beta), mode, _ptr(log_alpha), _ptr(S0), _ptr(o),
                                     _ptr(S_final), _stream(stream))
    if st != GDR_OK:
        raise GdrError(st, "gdr_fwd_chunked_noalloc")
    return o, S_final


class FwdChunkedCall:
    """One gdr_fwd_chunked call, checked and allocated once, to be enqueued
    any number of times on the same tensors (a training or serving loop with
    fixed shapes): calling it repeats the C call with the stored pointers and
    stream, without the per-call Python checks.  The tensors must stay alive
    and in place; ``o`` and ``S_final`` hold the results after each call."""

    def __init__(self, q, k, v, beta, log_alpha=None, S0=None, chunk: int = 64, *, o=None,
                 S_final=None, write_final: bool = True, workspace=None, stream=None,
                 prologue: int = 0):
        self._fn, self._args, self._name, (self.o, self.S_final), self.workspace = \
            _prepare_fwd_chunked(q, k, v, beta, log_alpha, S0, chunk, o, S_final, write_final,
                                 workspace, stream, prologue)
        self._keep = (q, k, v, beta, log_alpha, S0)   # the pointers stay valid

    def __call__(self):
        st = self._fn(*self._args)
        if st != GDR_OK:
            raise GdrError(st, self._name)
        return self.o, self.S_final


def gdr_bwd_chunked_workspace_size(B, H, L, d_k, d_v, C, dtype, alpha_mode) -> int:
    return int(load_library().gdr_bwd_chunked_workspace_size(B, H, L, d_k, d_v, C, dtype,
                                                             alpha_mode))


def _bwd_workspace(B, H, L, dk, dv, chunk, code, mode, workspace, dev):
    need = gdr_bwd_chunked_workspace_size(B, H, L, dk, dv, chunk, code, mode)
    if need == ctypes.c_size_t(-1).value:
        raise GdrError(GDR_ERR_UNSUPPORTED, "gdr_bwd_chunked_workspace_size")
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    return workspace, 0 if workspace is None else workspace.numel() * workspace.element_size()


def gdr_fwd_chunked_keep(q, k, v, beta, log_alpha=None, S0=None, chunk: int = 64, *, o=None,
                         S_final=None, write_final: bool = True, workspace=None, stream=None):
    """The forward of a training step: gdr_fwd_chunked's results, plus what
    the backward would recompute, kept in a backward workspace (allocated
    here unless given).  Returns (o, S_final or None, workspace); pass the
    workspace to gdr_bwd_chunked(..., kept=True)."""
    lib = load_library()
    if q.dim() != 4:
        raise ValueError("q must be [B, H, L, d_k]")
    B, H, L, dk = q.shape
    dv = v.shape[-1]
    dev, dt = q.device, q.dtype
    code = _dtype_code(dt)
    mode = _mode_of(log_alpha, q)
    _check(q, "q", dt, dev, (B, H, L, dk))
    _check(k, "k", dt, dev, (B, H, L, dk))
    _check(v, "v", dt, dev, (B, H, L, dv))
    _check(beta, "beta", torch.float32, dev, (B, H, L))
    if mode == GDR_ALPHA_SCALAR:
        _check(log_alpha, "log_alpha", torch.float32, dev, (B, H, L))
    elif mode == GDR_ALPHA_CHANNEL:
        _check(log_alpha, "log_alpha", torch.float32, dev, (B, H, L, dk))
    _check(S0, "S0", torch.float32, dev, (B, H, dv, dk))
    if o is None:
        o = torch.empty((B, H, L, dv), dtype=dt, device=dev)
    _check(o, "o", dt, dev, (B, H, L, dv))
    if S_final is None and write_final:
        S_final = torch.empty((B, H, dv, dk), dtype=torch.float32, device=dev)
    _check(S_final, "S_final", torch.float32, dev, (B, H, dv, dk))
    workspace, ws_bytes = _bwd_workspace(B, H, L, dk, dv, chunk, code, mode, workspace, dev)
    st = lib.gdr_fwd_chunked_keep(B, H, L, dk, dv, chunk, code, _ptr(q), _ptr(k), _ptr(v), _ptr(beta),
                                  mode, _ptr(log_alpha), _ptr(S0), _ptr(o), _ptr(S_final),
                                  _ptr(workspace), ws_bytes, _stream(stream))
    if st != GDR_OK:
        raise GdrError(st, "gdr_fwd_chunked_keep")
    return o, S_final, workspace


def gdr_bwd_chunked(q, k, v, beta, log_alpha, S0, dO, dS_final=None, chunk: int = 64, *,
                    want_dS0: bool = True, workspace=None, stream=None, kept: bool = False):
    """Gradients of gdr_fwd_chunked for output gradient dO [B,H,L,dv] (dtype
    of q) and final-state gradient dS_final (None | [B,H,dv,dk] fp32).
    Returns a dict of dq, dk, dv (dtype of q), dbeta, dlog_alpha (None for
    alpha = 1, else the shape of log_alpha) and dS0 (fp32, or None).
    kept=True: ``workspace`` is the one gdr_fwd_chunked_keep returned for the
    same inputs, and the forward is not recomputed (gdr_bwd_chunked_kept)."""
    if kept and workspace is None:
        raise ValueError("kept=True needs the workspace gdr_fwd_chunked_keep filled")
    lib = load_library()
    if q.dim() != 4:
        raise ValueError("q must be [B, H, L, d_k]")
    B, H, L, dk = q.shape
    dv = v.shape[-1]
    dev, dt = q.device, q.dtype
    code = _dtype_code(dt)
    mode = _mode_of(log_alpha, q)
    _check(q, "q", dt, dev, (B, H, L, dk))
    _check(k, "k", dt, dev, (B, H, L, dk))
    _check(v, "v", dt, dev, (B, H, L, dv))
    _check(beta, "beta", torch.float32, dev, (B, H, L))
    if mode == GDR_ALPHA_SCALAR:
        _check(log_alpha, "log_alpha", torch.float32, dev, (B, H, L))
    elif mode == GDR_ALPHA_CHANNEL:
        _check(log_alpha, "log_alpha", torch.float32, dev, (B, H, L, dk))
    _check(S0, "S0", torch.float32, dev, (B, H, dv, dk))
    _check(dO, "dO", dt, dev, (B, H, L, dv))
    _check(dS_final, "dS_final", torch.float32, dev, (B, H, dv, dk))
    g = dict(dq=torch.empty_like(q), dk=torch.empty_like(k), dv=torch.empty_like(v),
             dbeta=torch.empty_like(beta),
             dlog_alpha=None if log_alpha is None else torch.empty_like(log_alpha),
             dS0=torch.empty((B, H, dv, dk), dtype=torch.float32, device=dev) if want_dS0 else None)
    workspace, ws_bytes = _bwd_workspace(B, H, L, dk, dv, chunk, code, mode, workspace, dev)
    fn, name = (lib.gdr_bwd_chunked_kept, "gdr_bwd_chunked_kept") if kept else (lib.gdr_bwd_chunked,
                                                                                "gdr_bwd_chunked")
    st = fn(B, H, L, dk, dv, chunk, code, _ptr(q), _ptr(k), _ptr(v), _ptr(beta), mode, _ptr(log_alpha),
            _ptr(S0), _ptr(dO), _ptr(dS_final), _ptr(g["dq"]), _ptr(g["dk"]), _ptr(g["dv"]),
            _ptr(g["dbeta"]), _ptr(g["dlog_alpha"]), _ptr(g["dS0"]), _ptr(workspace), ws_bytes,
            _stream(stream))
    if st != GDR_OK:
        raise GdrError(st, name)
    return g


def gdr_fwd_varlen_workspace_size(N, H, T, d_k, d_v, C, dtype, alpha_mode) -> int:
    return int(load_library().gdr_fwd_varlen_workspace_size(N, H, T, d_k, d_v, C, dtype,
                                                            alpha_mode))


def gdr_fwd_varlen(q, k, v, beta, log_alpha, S0, cu_seqlens, chunk: int = 64, *, o=None,
                   S_final=None, write_final: bool = True, workspace=None, stream=None,
                   prologue: int = 0):
    """Chunkwise forward over a packed batch of N sequences.  q, k [H,T,dk];
    v [H,T,dv] (bf16 or fp32); beta [H,T] fp32; log_alpha None | [H,T] |
    [H,T,dk] fp32; cu_seqlens int32 GPU tensor [N+1] (cumulative offsets);
    S0 None | [N,H,dv,dk] fp32.  Returns (o [H,T,dv], S_final [N,H,dv,dk] or
    None)."""
    lib = load_library()
    if q.dim() != 3:
        raise ValueError("q must be [H, T, d_k]")
    H, T, dk = q.shape
    dv = v.shape[-1]
    dev, dt = q.device, q.dtype
    code = _dtype_code(dt)
    if log_alpha is None:
        mode = GDR_ALPHA_NONE
    else:
        mode = GDR_ALPHA_CHANNEL if log_alpha.dim() == 3 else GDR_ALPHA_SCALAR
    if cu_seqlens.dim() != 1 or cu_seqlens.numel() < 1:
        raise ValueError("cu_seqlens must be [N + 1]")
    N = cu_seqlens.numel() - 1
    _check(cu_seqlens, "cu_seqlens", torch.int32, dev, (N + 1,))
    _check(q, "q", dt, dev, (H, T, dk))
    _check(k, "k", dt, dev, (H, T, dk))
    _check(v, "v", dt, dev, (H, T, dv))
    _check(beta, "beta", torch.float32, dev, (H, T))
    if mode == GDR_ALPHA_SCALAR:
        _check(log_alpha, "log_alpha", torch.float32, dev, (H, T))
    elif mode == GDR_ALPHA_CHANNEL:
        _check(log_alpha, "log_alpha", torch.float32, dev, (H, T, dk))
    _check(S0, "S0", torch.float32, dev, (N, H, dv, dk))
    if o is None:
        o = torch.empty((H, T, dv), dtype=dt, device=dev)
    _check(o, "o", dt, dev, (H, T, dv))
    if S_final is None and write_final:
        S_final = torch.empty((N, H, dv, dk), dtype=torch.float32, device=dev)
    _check(S_final, "S_final", torch.float32, dev, (N, H, dv, dk))
    need = gdr_fwd_varlen_workspace_size(N, H, T, dk, dv, chunk, code, mode)
    if need == ctypes.c_size_t(-1).value:
        raise GdrError(GDR_ERR_UNSUPPORTED, "gdr_fwd_varlen_workspace_size")
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.gdr_fwd_varlen(N, H, T, _ptr(cu_seqlens), dk, dv, chunk, code, _ptr(q), _ptr(k),
                            _ptr(v), _ptr(beta), mode, _ptr(log_alpha), _ptr(S0), _ptr(o),
                            _ptr(S_final), _ptr(workspace), ws_bytes, _stream(stream),
                            int(prologue))
    if st != GDR_OK:
        raise GdrError(st, "gdr_fwd_varlen")
    return o, S_final


def gdr_decode_step(q, k, v, beta, log_alpha, S, o=None, *, stream=None, prologue: int = 0):
    """One decode step.  q, k [N,H,dk]; v [N,H,dv]; beta [N,H];
    log_alpha None | [N,H] | [N,H,dk]; S [N,H,dv,dk] fp32 (updated in
    place).  Returns o [N,H,dv].  ``prologue`` as for gdr_fwd_chunked."""
    lib = load_library()
    if q.dim() != 3:
        raise ValueError("q must be [N, H, d_k]")
    N, H, dk = q.shape
    dv = v.shape[-1]
    dev, dt = q.device, q.dtype
    code = _dtype_code(dt)
    mode = _mode_of(log_alpha, q)
    _check(q, "q", dt, dev, (N, H, dk))
    _check(k, "k", dt, dev, (N, H, dk))
    _check(v, "v", dt, dev, (N, H, dv))
    _check(beta, "beta", torch.float32, dev, (N, H))
    if mode == GDR_ALPHA_SCALAR:
        _check(log_alpha, "log_alpha", torch.float32, dev, (N, H))
    elif mode == GDR_ALPHA_CHANNEL:
        _check(log_alpha, "log_alpha", torch.float32, dev, (N, H, dk))
    _check(S, "S", torch.float32, dev, (N, H, dv, dk))
    if o is None:
        o = torch.empty((N, H, dv), dtype=dt, device=dev)
    _check(o, "o", dt, dev, (N, H, dv))
    args = (N, H, dk, dv, code, _ptr(q), _ptr(k), _ptr(v), _ptr(beta), mode, _ptr(log_alpha),
            _ptr(S), _ptr(o), _stream(stream))
    if prologue:
        st, name = lib.gdr_decode_step_ex(*args, int(prologue)), "gdr_decode_step_ex"
    else:
        st, name = lib.gdr_decode_step(*args), "gdr_decode_step"
    if st != GDR_OK:
        raise GdrError(st, name)
    return o
