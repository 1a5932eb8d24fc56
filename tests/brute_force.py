"""Independent fp64 references that pin the oracle (CPU, numpy).

Each function computes the same quantity as the oracle by a *different*
route, so that a slip in the oracle's loop (a dropped term, a wrong sign or
index, a transposed operand) shows up as a mismatch:

* ``masked_parallel_no_delta`` -- the parallel masked form of (gated) linear
  attention, O = (Q K^T . Gamma . M) diag(beta) V plus the decayed read of
  the initial state ("Chunkwise Parallel Form" and "Standard Softmax
  Attention" sections of the blog post "linear attention and its gated
  descendants": with the delta term removed and alpha = beta = 1 it is
  exactly (Q K^T . M) V with the causal mask including the diagonal).
* ``dense_transition`` -- the multiplicative form S_t = S_{t-1} A_t +
  beta_t v_t k_t^T with the explicit d_k x d_k transition matrix
  A_t = Diag(alpha_t)(I - beta_t k_t k_t^T) (blog post, end of the "Kimi
  Delta Attention" section, written here in the d_v x d_k orientation).
* ``kimi_orientation`` -- the recurrence exactly as the blog's Kimi section
  writes it, in the transposed d_k x d_v orientation:
  S'_t = (I - beta k k^T) Diag(alpha) S'_{t-1} + beta k v^T, o = S'^T q.
* ``mutant_loop`` -- a plain loop with switchable, deliberately planted
  mistakes; the pin tests check that every planted mistake fails at least
  one pin.
"""
from __future__ import annotations

import numpy as np


def _decay(log_alpha, L, dk, t):
    if log_alpha is None:
        return np.ones(dk)
    la = np.asarray(log_alpha, dtype=np.float64)
    if la.ndim == 1:
        return np.full(dk, np.exp(la[t]))
    return np.exp(la[t])


def masked_parallel_no_delta(q, k, v, beta, log_alpha=None, S0=None):
    """One chain (q,k [L,dk], v [L,dv]); returns o [L,dv] in O(L^2 d)."""
    q, k, v, beta = (np.asarray(x, dtype=np.float64) for x in (q, k, v, beta))
    L, dk = q.shape
    if log_alpha is None:
        G = np.zeros((L, dk))
    else:
        la = np.asarray(log_alpha, dtype=np.float64)
        G = np.cumsum(la if la.ndim == 2 else np.repeat(la[:, None], dk, axis=1), axis=0)
    # scores[r, i] = sum_c q[r,c] k[i,c] exp(G[r,c] - G[i,c]) for i <= r
    diff = G[:, None, :] - G[None, :, :]                    # [r, i, c]
    mask = np.tril(np.ones((L, L), dtype=bool))
    dec = np.where(mask[:, :, None], np.exp(np.where(mask[:, :, None], diff, 0.0)), 0.0)
    scores = np.einsum("rc,ic,ric->ri", q, k, dec)
    o = scores @ (beta[:, None] * v)
    if S0 is not None:
        S0 = np.asarray(S0, dtype=np.float64)
        o = o + (q * np.exp(G)) @ S0.T
    return o


def dense_transition(q, k, v, beta, log_alpha=None, S0=None):
    """One chain via explicit transition matrices; returns (o, S_final)."""
    q, k, v, beta = (np.asarray(x, dtype=np.float64) for x in (q, k, v, beta))
    L, dk = q.shape
    dv = v.shape[1]
    S = np.zeros((dv, dk)) if S0 is None else np.array(S0, dtype=np.float64)
    o = np.zeros((L, dv))
    eye = np.eye(dk)
    for t in range(L):
        A = np.diag(_decay(log_alpha, L, dk, t)) @ (eye - beta[t] * np.outer(k[t], k[t]))
        S = S @ A + beta[t] * np.outer(v[t], k[t])
        o[t] = S @ q[t]
    return o, S


def kimi_orientation(q, k, v, beta, log_alpha=None, S0=None):
    """One chain in the d_k x d_v orientation; returns (o, S'^T_final)."""
    q, k, v, beta = (np.asarray(x, dtype=np.float64) for x in (q, k, v, beta))
    L, dk = q.shape
    dv = v.shape[1]
    Sp = np.zeros((dk, dv)) if S0 is None else np.array(S0, dtype=np.float64).T.copy()
    o = np.zeros((L, dv))
    eye = np.eye(dk)
    for t in range(L):
        Sp = (eye - beta[t] * np.outer(k[t], k[t])) @ np.diag(_decay(log_alpha, L, dk, t)) @ Sp \
            + beta[t] * np.outer(k[t], v[t])
        o[t] = Sp.T @ q[t]
    return o, Sp.T


MUTATIONS = (
    "undecayed_prediction",   # predict from S_{t-1} instead of the decayed memory
    "read_before_write",      # o_t from the decayed memory before the write
    "decay_value_dim",        # Diag(alpha) on the left (value channels)
    "no_beta",                # residual not scaled by beta
    "residual_sign",          # v + pred instead of v - pred
    "transposed_read",        # o = S^T q
    "decay_after_write",      # alpha applied to (S + u k^T)
    "alpha_not_exponentiated",  # uses log alpha as the factor
    "shifted_gate",           # uses alpha_{t-1} at step t
)


def mutant_loop(q, k, v, beta, log_alpha=None, S0=None, mutation=None, no_delta=False):
    """Plain loop with one planted mistake (or none); returns (o, S)."""
    q, k, v, beta = (np.asarray(x, dtype=np.float64) for x in (q, k, v, beta))
    L, dk = q.shape
    dv = v.shape[1]
    S = np.zeros((dv, dk)) if S0 is None else np.array(S0, dtype=np.float64)
    o = np.zeros((L, dv))
    for t in range(L):
        tt = max(t - 1, 0) if mutation == "shifted_gate" else t
        if mutation == "alpha_not_exponentiated" and log_alpha is not None:
            la = np.asarray(log_alpha, dtype=np.float64)
            a = np.full(dk, la[tt]) if la.ndim == 1 else la[tt]
        else:
            a = _decay(log_alpha, L, dk, tt)
        if mutation == "decay_value_dim":
            Sbar = (a[:dv, None] if dv <= dk else np.resize(a, dv)[:, None]) * S
        elif mutation == "decay_after_write":
            Sbar = S
        else:
            Sbar = S * a[None, :]
        pred = (S if mutation == "undecayed_prediction" else Sbar) @ k[t]
        if no_delta:
            pred = np.zeros(dv)
        if mutation == "residual_sign":
            u = beta[t] * (v[t] + pred)
        elif mutation == "no_beta":
            u = v[t] - pred
        else:
            u = beta[t] * (v[t] - pred)
        Snew = Sbar + np.outer(u, k[t])
        if mutation == "decay_after_write":
            Snew = Snew * a[None, :]
        src = Sbar if mutation == "read_before_write" else Snew
        o[t] = src.T @ q[t][:dv] if mutation == "transposed_read" else src @ q[t]
        S = Snew
    return o, S
