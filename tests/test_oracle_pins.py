"""Pins for the fp64 oracle (CPU only).

The oracle is trusted only because it agrees with things other than itself:
hand-worked examples, closed forms, invariants the pages state, and
independent brute-force routes (``brute_force.py``).  The last test plants
plausible mistakes in a separate loop and checks that every one of them
fails at least one pin, i.e. the pins are sensitive to such mistakes.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import pytest

import oracle
import brute_force as bf

NONE, SCALAR, CHANNEL = oracle.ALPHA_NONE, oracle.ALPHA_SCALAR, oracle.ALPHA_CHANNEL
GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")


# --------------------------------------------------------------------------
# helpers
def _unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _rand_chain(rng, L, dk, dv, mode, s0=True, shift=1.0):
    q = _unit(rng.standard_normal((L, dk)))
    k = _unit(rng.standard_normal((L, dk)))
    v = rng.standard_normal((L, dv))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal(L)))
    if mode == NONE:
        la = None
    elif mode == SCALAR:
        la = -np.log1p(np.exp(rng.standard_normal(L) + shift))
    else:
        la = -np.log1p(np.exp(rng.standard_normal((L, dk)) + shift))
    S0 = 0.3 * rng.standard_normal((dv, dk)) if s0 else None
    return q, k, v, beta, la, S0


def oracle_runner(q, k, v, beta, la=None, S0=None, no_delta=False):
    mode = NONE if la is None else (CHANNEL if np.ndim(la) == 2 else SCALAR)
    return oracle.run(q, k, v, beta, la, S0, mode=mode, no_delta=no_delta, nthreads=1)


def _err(a, b):
    a, b = np.asarray(a), np.asarray(b)
    return float(np.max(np.abs(a - b))) / max(1.0, float(np.max(np.abs(b))))


# --------------------------------------------------------------------------
# pins, each written against an arbitrary runner so the mutation test can
# reuse them.  Each returns the worst error it saw; the bound is 1e-10.
def pin_exact_recall(run):
    """alpha = beta = 1, orthonormal keys: S k_i = v_i, and querying with k_i
    returns v_i ("DeltaNet" section of the blog post: perfectly orthogonal
    keys isolate v_j; beta = 1 fully replaces the retrieved value)."""
    rng = np.random.default_rng(11)
    dk, dv, n = 8, 5, 6
    Qm, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    keys = Qm.T[:n]                                  # orthonormal rows
    vals = rng.standard_normal((n, dv))
    L = 2 * n
    k = np.vstack([keys, _unit(rng.standard_normal((n, dk)))])
    v = np.vstack([vals, rng.standard_normal((n, dv))])
    q = np.vstack([_unit(rng.standard_normal((n, dk))), keys])
    beta = np.concatenate([np.ones(n), np.zeros(n)])  # write n pairs, then only read
    worst = 0.0
    for la in (None, np.zeros(L)):
        o, S = run(q, k, v, beta, la, None)
        worst = max(worst, _err(o[n:], vals), _err(S @ keys.T, vals.T))
    return worst


def pin_overwrite(run):
    """The same orthonormal keys written twice: the memory returns the most
    recent value (beta = 1 full replacement, blog "DeltaNet" section)."""
    rng = np.random.default_rng(12)
    dk, dv, n = 6, 4, 4
    Qm, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    keys = Qm.T[:n]
    v1, v2 = rng.standard_normal((n, dv)), rng.standard_normal((n, dv))
    k = np.vstack([keys, keys[::-1]])
    v = np.vstack([v1, v2[::-1]])
    q = _unit(rng.standard_normal((2 * n, dk)))
    o, S = run(q, k, v, np.ones(2 * n), None, 0.5 * rng.standard_normal((dv, dk)))
    # S0 components outside span(keys) survive; the key directions hold v2.
    return _err(S @ keys.T, v2.T)


def pin_beta_one_write(run):
    """beta = 1 and a unit key: after the write S_t k_t = v_t exactly, for any
    decay and any (non-orthogonal) history (the delta rule as one SGD step on
    0.5 |S k - v|^2 with unit step, wiki "DeltaNet" item).  With q_t = k_t the
    output is v_t."""
    rng = np.random.default_rng(13)
    worst = 0.0
    for mode in (NONE, SCALAR, CHANNEL):
        q, k, v, beta, la, S0 = _rand_chain(rng, 20, 7, 5, mode)
        o, _ = run(k, k, v, np.ones(20), la, S0)
        worst = max(worst, _err(o, v))
    return worst


def pin_beta_zero(run):
    """beta = 0 keeps memory apart from the decay (blog "DeltaNet": beta = 0
    keeps old memory): o_t = S0 (prod alpha . q_t); S_final = S0 Diag(prod)."""
    rng = np.random.default_rng(14)
    worst = 0.0
    for mode in (NONE, SCALAR, CHANNEL):
        q, k, v, _, la, S0 = _rand_chain(rng, 12, 6, 4, mode, shift=-1.0)
        o, S = run(q, k, v, np.zeros(12), la, S0)
        if la is None:
            cum = np.zeros((12, 6))
        else:
            la2 = la if np.ndim(la) == 2 else np.repeat(la[:, None], 6, axis=1)
            cum = np.cumsum(la2, axis=0)
        ref = (q * np.exp(cum)) @ S0.T
        worst = max(worst, _err(o, ref), _err(S, S0 * np.exp(cum[-1])[None, :]))
    return worst


def pin_first_token(run):
    """From a zero state one token gives S_1 = beta v k^T and
    o_1 = beta (k.q) v (blog "DeltaNet" update with S_0 = 0)."""
    rng = np.random.default_rng(15)
    worst = 0.0
    for mode in (NONE, SCALAR, CHANNEL):
        q, k, v, beta, la, _ = _rand_chain(rng, 1, 5, 3, mode)
        o, S = run(q, k, v, beta, la, None)
        worst = max(worst, _err(o[0], beta[0] * (k[0] @ q[0]) * v[0]),
                    _err(S, beta[0] * np.outer(v[0], k[0])))
    return worst


def pin_linear_attention_sum(run):
    """Delta term removed, alpha = beta = 1: S_L = sum_i v_i k_i^T = V^T K
    (blog "Linear Attention as a Linear RNN")."""
    rng = np.random.default_rng(16)
    q, k, v, _, _, _ = _rand_chain(rng, 30, 6, 4, NONE)
    o, S = run(q, k, v, np.ones(30), None, None, no_delta=True)
    return max(_err(S, v.T @ k), _err(o, np.tril(q @ k.T) @ v))


def pin_masked_parallel(run):
    """Delta term removed: the loop equals the parallel masked form, with
    decay and beta, for every gate mode (blog "Chunkwise Parallel Form")."""
    rng = np.random.default_rng(17)
    worst = 0.0
    for mode in (NONE, SCALAR, CHANNEL):
        q, k, v, beta, la, S0 = _rand_chain(rng, 40, 6, 5, mode, shift=0.0)
        o, _ = run(q, k, v, beta, la, S0, no_delta=True)
        worst = max(worst, _err(o, bf.masked_parallel_no_delta(q, k, v, beta, la, S0)))
    return worst


def pin_dense_transition(run):
    """Explicit d_k x d_k transitions A_t = Diag(alpha)(I - beta k k^T) (blog,
    end of the "Kimi Delta Attention" section), all gate modes."""
    rng = np.random.default_rng(18)
    worst = 0.0
    for mode in (NONE, SCALAR, CHANNEL):
        q, k, v, beta, la, S0 = _rand_chain(rng, 24, 6, 6, mode, shift=-0.5)
        o, S = run(q, k, v, beta, la, S0)
        ro, rS = bf.dense_transition(q, k, v, beta, la, S0)
        worst = max(worst, _err(o, ro), _err(S, rS))
    return worst


def pin_kimi_orientation(run):
    """The blog's Kimi recurrence in the d_k x d_v orientation gives the
    transposed state and the same outputs (orientation reading)."""
    rng = np.random.default_rng(19)
    worst = 0.0
    for mode in (NONE, SCALAR, CHANNEL):
        q, k, v, beta, la, S0 = _rand_chain(rng, 24, 6, 6, mode, shift=-0.5)
        o, S = run(q, k, v, beta, la, S0)
        ro, rS = bf.kimi_orientation(q, k, v, beta, la, S0)
        worst = max(worst, _err(o, ro), _err(S, rS))
    return worst


def pin_mode_reductions(run):
    """Channel gate with equal channels == scalar gate; scalar gate with
    log alpha = 0 == DeltaNet ("Linear Attention Architectures", Sec. 3:
    if the vector gate collapses to a scalar the update reduces to Gated
    DeltaNet's; blog: Gated DeltaNet adds a decay to DeltaNet)."""
    rng = np.random.default_rng(20)
    q, k, v, beta, la, S0 = _rand_chain(rng, 30, 6, 4, SCALAR)
    o_s, S_s = run(q, k, v, beta, la, S0)
    o_c, S_c = run(q, k, v, beta, np.repeat(la[:, None], 6, axis=1), S0)
    o_n, S_n = run(q, k, v, beta, None, S0)
    o_z, S_z = run(q, k, v, beta, np.zeros(30), S0)
    return max(_err(o_c, o_s), _err(S_c, S_s), _err(o_z, o_n), _err(S_z, S_n))


def pin_resume(run):
    """The state is the whole memory: running L1 tokens, then L2 tokens from
    the resulting state equals one run of L1 + L2 tokens (blog "Chunkwise
    Parallel Form": the state is additive across boundaries; "Recurrent
    Linear Attention for Inference": one O(d^2) state)."""
    rng = np.random.default_rng(21)
    worst = 0.0
    for mode in (NONE, SCALAR, CHANNEL):
        q, k, v, beta, la, S0 = _rand_chain(rng, 37, 6, 5, mode)
        o, S = run(q, k, v, beta, la, S0)
        cut = 16
        la1 = None if la is None else la[:cut]
        la2 = None if la is None else la[cut:]
        o1, S1 = run(q[:cut], k[:cut], v[:cut], beta[:cut], la1, S0)
        o2, S2 = run(q[cut:], k[cut:], v[cut:], beta[cut:], la2, S1)
        worst = max(worst, _err(np.vstack([o1, o2]), o), _err(S2, S))
    return worst


def _golden_value(x):
    if isinstance(x, str):
        sign = -1.0 if x.startswith("-") else 1.0
        return sign * math.log(float(x.lstrip("-").replace("ln", "")))
    return float(x)


def _golden_array(a):
    if a is None:
        return None
    if isinstance(a, list):
        return np.array([_golden_array(x) for x in a], dtype=np.float64)
    return _golden_value(a)


def pin_worked_examples(run):
    """Hand-worked 2x2 examples (tests/golden/worked_examples.json)."""
    with open(GOLDEN) as f:
        ex = json.load(f)["examples"]
    worst = 0.0
    for e in ex:
        args = [_golden_array(e[n]) for n in ("q", "k", "v", "beta", "log_alpha", "S0")]
        o, S = run(*args)
        worst = max(worst, _err(o, _golden_array(e["o"])), _err(S, _golden_array(e["S_final"])))
    return worst


PINS = [pin_exact_recall, pin_overwrite, pin_beta_one_write, pin_beta_zero, pin_first_token,
        pin_linear_attention_sum, pin_masked_parallel, pin_dense_transition,
        pin_kimi_orientation, pin_mode_reductions, pin_resume, pin_worked_examples]
TOL = 1e-10


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_oracle_pin(pin):
    assert pin(oracle_runner) <= TOL


@pytest.mark.parametrize("mutation", bf.MUTATIONS)
def test_planted_mistake_is_caught(mutation):
    """Every planted mistake fails at least one pin (pins are sensitive)."""
    def run(q, k, v, beta, la=None, S0=None, no_delta=False):
        return bf.mutant_loop(q, k, v, beta, la, S0, mutation=mutation, no_delta=no_delta)

    failed = []
    for pin in PINS:
        try:
            e = pin(run)
            if not (e <= TOL):
                failed.append(pin.__name__)
        except (ValueError, IndexError):
            failed.append(pin.__name__)
    assert failed, f"mutation {mutation} passed every pin"


def test_unmutated_loop_passes_pins():
    def run(q, k, v, beta, la=None, S0=None, no_delta=False):
        return bf.mutant_loop(q, k, v, beta, la, S0, mutation=None, no_delta=no_delta)

    for pin in PINS:
        assert pin(run) <= TOL, pin.__name__


def test_state_size_constant_in_length():
    """The memory is one d_v x d_k matrix per chain whatever L is (blog
    "Recurrent Linear Attention for Inference": O(d^2) memory)."""
    rng = np.random.default_rng(22)
    for L in (1, 64, 4096):
        q, k, v, beta, la, S0 = _rand_chain(rng, L, 8, 4, SCALAR)
        o, S = oracle.run(q[None], k[None], v[None], beta[None], la[None], S0[None])
        assert S.shape == (1, 4, 8) and o.shape == (1, L, 4)


def test_batched_chains_are_independent():
    """Leading (batch, head) axes are independent chains: running them
    together equals running each alone (blog: each head runs its own
    recurrent state update)."""
    rng = np.random.default_rng(23)
    chains = [_rand_chain(rng, 19, 5, 3, CHANNEL) for _ in range(6)]
    stack = [np.stack([c[i] for c in chains]).reshape((2, 3) + np.shape(chains[0][i]))
             for i in range(6)]
    o, S = oracle.run(*stack, nthreads=3)
    for j, c in enumerate(chains):
        oj, Sj = oracle_runner(*c)
        b, h = divmod(j, 3)
        assert np.array_equal(o[b, h], oj) and np.array_equal(S[b, h], Sj)


def test_oracle_rejects_bad_shapes():
    rng = np.random.default_rng(24)
    q, k, v, beta, la, S0 = _rand_chain(rng, 5, 4, 3, SCALAR)
    with pytest.raises(ValueError):
        oracle.run(q, k[:4], v, beta, la, S0)
    with pytest.raises(ValueError):
        oracle.run(q, k, v, beta, la[:3], S0, mode=SCALAR)


# --------------------------------------------------------------------------
# the input-side prologue (unit-norm q, k; sigmoid gates)
def test_prologue_gates_closed_forms():
    """sigmoid and log-sigmoid at points with exact values, and in both far
    tails, where a naive exp(-x) would overflow."""
    ln3 = math.log(3.0)
    s = oracle.sigmoid(np.array([0.0, ln3, -ln3, 800.0, -800.0]))
    assert np.allclose(s[:3], [0.5, 0.75, 0.25], rtol=1e-15, atol=0)
    assert s[3] == 1.0 and 0.0 <= s[4] < 1e-300
    ls = oracle.log_sigmoid(np.array([0.0, ln3, -ln3, 800.0, -800.0]))
    assert np.allclose(ls[:3], [-math.log(2.0), math.log(0.75), math.log(0.25)], rtol=1e-15, atol=0)
    assert ls[3] == 0.0 and ls[4] == -800.0


def test_prologue_gates_against_scipy():
    """The gates agree with scipy's expit / log_expit (independent routines)
    over the range a gate pre-activation takes, and obey
    sigmoid(x) + sigmoid(-x) = 1 and exp(log_sigmoid(x)) = sigmoid(x)."""
    from scipy import special
    x = np.linspace(-60.0, 60.0, 4801)
    assert np.max(np.abs(oracle.sigmoid(x) - special.expit(x)) / special.expit(x)) < 1e-14
    assert np.max(np.abs(oracle.log_sigmoid(x) - special.log_expit(x))
                  / np.maximum(np.abs(special.log_expit(x)), 1e-300)) < 1e-13
    assert np.max(np.abs(oracle.sigmoid(x) + oracle.sigmoid(-x) - 1.0)) < 1e-15
    assert np.max(np.abs(np.exp(oracle.log_sigmoid(x)) - oracle.sigmoid(x))) < 1e-15


def test_prologue_norm_closed_forms():
    x = np.array([[3.0, 4.0, 0.0], [0.0, 0.0, 0.0], [1e-9, 0.0, 0.0], [0.0, -2.0, 0.0]])
    y = oracle.l2_normalise(x)
    assert np.array_equal(y[0], [0.6, 0.8, 0.0])
    assert np.array_equal(y[1], [0.0, 0.0, 0.0])           # zero stays zero
    assert np.allclose(y[2], [1e-3, 0.0, 0.0], rtol=1e-15)  # below the 1e-6 floor
    assert np.array_equal(y[3], [0.0, -1.0, 0.0])
    rng = np.random.default_rng(31)
    z = rng.standard_normal((50, 128)) * rng.lognormal(0.0, 2.0, (50, 1))
    assert np.max(np.abs(np.linalg.norm(oracle.l2_normalise(z), axis=-1) - 1.0)) < 1e-14
    assert np.max(np.abs(oracle.l2_normalise(7.5 * z) - oracle.l2_normalise(z))) < 1e-15


def test_prologue_feeds_the_recurrence():
    """run(raw, pro=3) equals the recurrence on inputs activated by
    independent routines (numpy's norm, scipy's expit / log_expit), for every
    gate mode; each flag alone touches only its own inputs."""
    from scipy import special
    rng = np.random.default_rng(32)
    for mode in (NONE, SCALAR, CHANNEL):
        L, dk, dv = 23, 8, 5
        q = rng.standard_normal((L, dk)) * rng.lognormal(0.0, 1.0, (L, 1))
        k = rng.standard_normal((L, dk)) * rng.lognormal(0.0, 1.0, (L, 1))
        v = rng.standard_normal((L, dv))
        b = rng.standard_normal(L)
        a = None if mode == NONE else rng.standard_normal((L,) if mode == SCALAR else (L, dk)) + 2.0
        S0 = 0.3 * rng.standard_normal((dv, dk))
        qn = q / np.linalg.norm(q, axis=-1, keepdims=True)
        kn = k / np.linalg.norm(k, axis=-1, keepdims=True)
        la = None if a is None else special.log_expit(a)
        ro, rS = oracle_runner(qn, kn, v, special.expit(b), la, S0)
        o, S = oracle.run(q, k, v, b, a, S0, mode=mode, pro=3, nthreads=1)
        assert _err(o, ro) < 1e-12 and _err(S, rS) < 1e-12
        o1, _ = oracle.run(q, k, v, special.expit(b), la, S0, mode=mode, pro=1, nthreads=1)
        assert _err(o1, ro) < 1e-12
        o2, _ = oracle.run(qn, kn, v, b, a, S0, mode=mode, pro=2, nthreads=1)
        assert _err(o2, ro) < 1e-12


def test_prologue_gate_signs():
    """alpha = sigmoid(a): a -> +inf keeps the memory (DeltaNet), a -> -inf
    empties it before every write, so with S0 = 0 each output is the lone
    write read back, o_t = beta_t v_t (k_t . q_t).  Swapping the sign of
    either gate fails one of the two."""
    rng = np.random.default_rng(33)
    L, dk, dv = 17, 6, 4
    q, k = _unit(rng.standard_normal((L, dk))), _unit(rng.standard_normal((L, dk)))
    v, b = rng.standard_normal((L, dv)), rng.standard_normal(L)
    beta = 1.0 / (1.0 + np.exp(-b))
    keep, _ = oracle.run(q, k, v, b, np.full(L, 60.0), None, mode=SCALAR, pro=2, nthreads=1)
    delta, _ = oracle_runner(q, k, v, beta)
    assert _err(keep, delta) < 1e-12
    gone, _ = oracle.run(q, k, v, b, np.full(L, -700.0), None, mode=SCALAR, pro=2, nthreads=1)
    lone = beta[:, None] * v * np.sum(k * q, axis=-1)[:, None]
    assert _err(gone, lone) < 1e-12


def test_prologue_norm_exact_recall():
    """With PRO_L2NORM_QK, orthogonal keys of any length and beta = 1 store
    each value exactly, and a query along a stored key (any length) reads
    that value back ("linear attention and its gated descendants",
    "DeltaNet": recall is exact for normalised, orthogonal keys).  Tokens
    0-3 write key t; tokens 4-7 (beta = 0, nothing written) read keys
    1, 3, 0, 2 back."""
    k = np.vstack([np.diag([5.0, 0.1, 2.0, 30.0]), np.full((4, 4), 9.0)])
    v = np.vstack([np.arange(12.0).reshape(4, 3) - 4.0, np.full((4, 3), 100.0)])
    perm = [1, 3, 0, 2]
    q = np.vstack([np.ones((4, 4)), np.diag([7.0, 0.02, 1.0, 3.0])[perm]])
    beta = np.array([1.0] * 4 + [0.0] * 4)
    o, S = oracle.run(q, k, v, beta, None, None, mode=NONE, pro=1, nthreads=1)
    assert _err(S, v[:4].T) < 1e-14
    assert _err(o[4:], v[perm]) < 1e-14
    # without the prologue the same raw keys store scaled, mixed values
    o_raw, _ = oracle.run(q, k, v, beta, None, None, mode=NONE, nthreads=1)
    assert _err(o_raw[4:], v[perm]) > 1e-3


def test_prologue_rejects_unknown_bits():
    x = np.zeros((2, 4))
    with pytest.raises(ValueError):
        oracle.prologue(x, x, np.zeros(2), None, 4)


# --------------------------------------------------------------------------
# gradients (reverse mode of the token recurrence)
def _fd_grads(loss, args, h=1e-6):
    """Central finite differences of loss(**args) for every array argument."""
    out = {}
    for name, x in args.items():
        if x is None:
            continue
        fd = np.zeros(np.shape(x))
        for idx in np.ndindex(fd.shape):
            xp, xm = np.array(x, dtype=np.float64), np.array(x, dtype=np.float64)
            xp[idx] += h
            xm[idx] -= h
            fd[idx] = (loss(**{**args, name: xp}) - loss(**{**args, name: xm})) / (2 * h)
        out[name] = fd
    return out


GRAD_NAMES = dict(q="dq", k="dk", v="dv", beta="dbeta", la="dlog_alpha", S0="dS0")


@pytest.mark.parametrize("mode", [NONE, SCALAR, CHANNEL])
def test_backward_matches_finite_differences(mode):
    """Every gradient of L = <o, do> + <S_final, dS_final> against central
    differences of the forward oracle, over 70 tokens (the backward keeps a
    state every 64 tokens and recomputes the rest)."""
    rng = np.random.default_rng(40 + mode)
    q, k, v, beta, la, S0 = _rand_chain(rng, 70, 5, 3, mode)
    do = rng.standard_normal((70, 3))
    dSf = rng.standard_normal((3, 5))

    def loss(q, k, v, beta, la, S0):
        o, S = oracle.run(q, k, v, beta, la, S0, mode=mode, nthreads=1)
        return float(np.sum(o * do) + np.sum(S * dSf))

    g = oracle.backward(q, k, v, beta, la, S0, do, dSf, mode=mode, nthreads=1)
    fd = _fd_grads(loss, dict(q=q, k=k, v=v, beta=beta, la=la, S0=S0))
    for name, ref in fd.items():
        got = g[GRAD_NAMES[name]]
        assert np.max(np.abs(got - ref)) / max(1.0, np.max(np.abs(ref))) < 1e-7, name
    if mode == NONE:
        assert g["dlog_alpha"] is None


def test_backward_first_token_closed_form():
    """L = 1 from S0: o = S_1 q with S_1 = a S0 + beta (v - a S0 k) k^T, so
    dv = beta (k.q) do, dq = S_1^T do, dk = beta (v - a S0 k).do q - beta a S0^T do (k.q),
    dbeta = (k.q) (v - a S0 k).do, dS0 = a do (q - beta (k.q) k)^T,
    dlog a = a <do (q - beta (k.q) k)^T, S0>."""
    rng = np.random.default_rng(41)
    dk_, dv_ = 6, 4
    q, k = _unit(rng.standard_normal(dk_)), _unit(rng.standard_normal(dk_))
    v, S0, do = rng.standard_normal(dv_), rng.standard_normal((dv_, dk_)), rng.standard_normal(dv_)
    b, la = 0.7, -0.4
    a = math.exp(la)
    r = v - a * S0 @ k
    S1 = a * S0 + b * np.outer(r, k)
    g = oracle.backward(q[None], k[None], v[None], np.array([b]), np.array([la]), S0, do[None],
                        None, mode=SCALAR, nthreads=1)
    kq = k @ q
    assert np.allclose(g["dv"][0], b * kq * do, atol=1e-13)
    assert np.allclose(g["dq"][0], S1.T @ do, atol=1e-13)
    assert np.allclose(g["dk"][0], b * (r @ do) * q - b * a * kq * (S0.T @ do), atol=1e-13)
    assert np.allclose(g["dbeta"][0], kq * (r @ do), atol=1e-13)
    w = q - b * kq * k
    assert np.allclose(g["dS0"], a * np.outer(do, w), atol=1e-13)
    assert np.allclose(g["dlog_alpha"][0], a * np.sum(np.outer(do, w) * S0), atol=1e-13)


@pytest.mark.parametrize("flags", [1, 2, 3])
def test_backward_through_the_prologue(flags):
    """Gradients with respect to raw q, k and gate pre-activations against
    finite differences of run(raw, pro=flags)."""
    rng = np.random.default_rng(42 + flags)
    L, dk_, dv_ = 9, 4, 3
    q = rng.standard_normal((L, dk_)) * 3.0
    k = rng.standard_normal((L, dk_)) * 0.5
    v = rng.standard_normal((L, dv_))
    b = rng.standard_normal(L)
    a = -(rng.standard_normal((L, dk_)) + 2.0)
    if not flags & 1:
        q, k = _unit(q), _unit(k)
    if not flags & 2:
        b, a = 1.0 / (1.0 + np.exp(-b)), -np.log1p(np.exp(-a))
    S0 = 0.3 * rng.standard_normal((dv_, dk_))
    do = rng.standard_normal((L, dv_))

    def loss(q, k, v, beta, la, S0):
        o, _ = oracle.run(q, k, v, beta, la, S0, mode=CHANNEL, pro=flags, nthreads=1)
        return float(np.sum(o * do))

    g = oracle.backward(q, k, v, b, a, S0, do, None, mode=CHANNEL, pro=flags, nthreads=1)
    fd = _fd_grads(loss, dict(q=q, k=k, v=v, beta=b, la=a, S0=S0))
    for name, ref in fd.items():
        got = g[GRAD_NAMES[name]]
        assert np.max(np.abs(got - ref)) / max(1.0, np.max(np.abs(ref))) < 1e-7, name


def test_backward_chains_are_independent():
    rng = np.random.default_rng(43)
    chains = [_rand_chain(rng, 11, 4, 3, SCALAR) for _ in range(4)]
    dos = [rng.standard_normal((11, 3)) for _ in range(4)]
    stack = lambda i: np.stack([c[i] for c in chains]).reshape((2, 2) + np.shape(chains[0][i]))
    g = oracle.backward(*[stack(i) for i in range(6)], np.stack(dos).reshape(2, 2, 11, 3), None,
                        nthreads=2)
    for j, c in enumerate(chains):
        gj = oracle.backward(*c, dos[j], None, mode=SCALAR, nthreads=1)
        for name in ("dq", "dk", "dv", "dbeta", "dlog_alpha", "dS0"):
            assert np.array_equal(g[name][j // 2, j % 2], gj[name]), name
