"""Pins of the oracle's gated variant (Gated EFLA).

The pages name a gated variant (papernotes note: main-results table, row
"Gated EFLA"; key findings: the exact flow upgrades Gated DeltaNet, and any
delta-rule variant, as an underlying algebraic change) but print no formula.
The reading pinned here: Gated DeltaNet's update with the exact-flow
coefficient, S_t = g_t (I - c_t k_t k_t^T) S_{t-1} + c_t k_t v_t^T with a
per-token decay g_t = exp(log_g_t), read out as o_t = S_t^T q_t.

Each test checks the oracle against something other than its own formula:
the exact ODE solution (scipy expm of the augmented system, 关键设计 items
1-2) applied to the decayed state, a closed form for mutually orthogonal keys,
pure decay with zero keys, a reset by a vanishing gate, reduction to the
ungated oracle, and an independent chunked (WY/UT) evaluation with the decays
carried inside each chunk, the form the GPU path uses.
"""
import math

import numpy as np
import pytest
import scipy.linalg

import oracle

RNG = np.random.default_rng(777)


def exact_update(S, k, v, beta):
    """Solution of dS/dt = -k k^T S + k v^T over [0, beta] from S (zero-order
    hold), via scipy's matrix exponential of the augmented linear system."""
    dk, dv = S.shape
    M = np.zeros((dk + dv, dk + dv))
    M[:dk, :dk] = -np.outer(k, k)
    M[:dk, dk:] = np.outer(k, v)
    return (scipy.linalg.expm(beta * M) @ np.vstack([S, np.eye(dv)]))[:dk]


def unit(d):
    g = RNG.standard_normal(d)
    return g / np.linalg.norm(g)


def test_gated_step_is_exact_flow_of_decayed_state():
    d, T = 5, 30
    S0 = RNG.standard_normal((d, d))
    q = RNG.standard_normal((T, d))
    k = np.stack([unit(d) * n for n in np.exp(RNG.uniform(math.log(0.3), math.log(6), T))])
    v = RNG.standard_normal((T, d))
    beta = RNG.uniform(0.1, 1.0, T)
    log_g = -RNG.uniform(0.0, 0.7, T)
    o, sf = oracle.fwd_gated(q[None], k[None], v[None], beta[None], log_g[None], S0[None])
    S = S0.copy()
    for t in range(T):
        S = exact_update(math.exp(log_g[t]) * S, k[t], v[t], beta[t])
        np.testing.assert_allclose(o[0, t], S.T @ q[t], rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(sf[0], S, rtol=1e-11, atol=1e-12)


def test_zero_log_decay_is_the_ungated_oracle():
    nh, T, d = 3, 41, 6
    q, k, v = (RNG.standard_normal((nh, T, d)) for _ in range(3))
    beta = RNG.uniform(0, 1, (nh, T))
    S0 = RNG.standard_normal((nh, d, d))
    for mode in (oracle.EXACT, oracle.EULER, oracle.RK4, oracle.ORDER2):
        og, sg = oracle.fwd_gated(q, k, v, beta, np.zeros((nh, T)), S0, mode=mode, nthreads=2)
        ou, su = oracle.fwd(q, k, v, beta, S0, mode=mode)
        # the two steps round in a different order (g (S - c k p^T) + c k v^T
        # against S + c k (v - p)^T); the Euler and RK4 steps grow the state on
        # these unscaled keys, so the bound is relative to each result's size
        np.testing.assert_allclose(og, ou, rtol=1e-12, atol=1e-12 * np.abs(ou).max())
        np.testing.assert_allclose(sg, su, rtol=1e-12, atol=1e-12 * np.abs(su).max())


def test_orthogonal_keys_closed_form():
    """Mutually orthogonal keys commute: S_T = G_T prod_t (I - c_t k_t k_t^T) S0 +
    sum_t (G_T / G_t) c_t k_t v_t^T with G_t = g_1 ... g_t, since each input
    term is left alone by the later, orthogonal transitions and only decays."""
    d = 6
    Qm, _ = np.linalg.qr(RNG.standard_normal((d, d)))
    norms = np.array([0.5, 1.0, 2.0, 3.0, 5.0, 9.0])
    k = (Qm.T * norms[:, None])
    T = d
    v = RNG.standard_normal((T, d))
    q = RNG.standard_normal((T, d))
    beta = RNG.uniform(0.2, 1.0, T)
    log_g = -RNG.uniform(0.0, 1.0, T)
    S0 = RNG.standard_normal((d, d))
    _, sf = oracle.fwd_gated(q[None], k[None], v[None], beta[None], log_g[None], S0[None])
    lam = norms ** 2
    c = -np.expm1(-beta * lam) / lam
    G = np.exp(np.cumsum(log_g))
    P = np.eye(d)
    for t in range(T):
        P = (np.eye(d) - c[t] * np.outer(k[t], k[t])) @ P
    want = G[-1] * P @ S0 + sum((G[-1] / G[t]) * c[t] * np.outer(k[t], v[t]) for t in range(T))
    np.testing.assert_allclose(sf[0], want, rtol=1e-12, atol=1e-12)


def test_zero_keys_decay_only_and_vanishing_gate_resets():
    d, T = 4, 12
    S0 = RNG.standard_normal((1, d, d))
    q, v = RNG.standard_normal((1, T, d)), RNG.standard_normal((1, T, d))
    beta = RNG.uniform(0, 1, (1, T))
    log_g = -RNG.uniform(0, 0.5, (1, T))
    o, sf = oracle.fwd_gated(q, np.zeros((1, T, d)), v, beta, log_g, S0)
    G = np.exp(np.cumsum(log_g[0]))
    np.testing.assert_allclose(sf[0], G[-1] * S0[0], rtol=1e-14)
    np.testing.assert_allclose(o[0], G[:, None] * (q[0] @ S0[0]), rtol=1e-13)
    # g_t = 0 at token t: the state before t is forgotten, S_t = c_t k_t v_t^T
    k = RNG.standard_normal((1, T, d))
    lg = log_g.copy()
    lg[0, 5] = -800.0  # exp underflows to exactly 0
    _, s5 = oracle.fwd_gated(q[:, :6], k[:, :6], v[:, :6], beta[:, :6], lg[:, :6], S0)
    lam = float(k[0, 5] @ k[0, 5])
    c = -math.expm1(-beta[0, 5] * lam) / lam
    np.testing.assert_allclose(s5[0], c * np.outer(k[0, 5], v[0, 5]), rtol=1e-13, atol=1e-15)


def chunked_gated(q, k, v, beta, log_g, S0, C):
    """Chunked (WY/UT) gated evaluation, numpy fp64, written from the
    recurrence: with b_r the cumulative log-decay inside a chunk
    (b_r = log_g_1 + ... + log_g_r) and Gamma_r = exp(b_r),
      A  = strictly-lower(diag(c) (K K^T) * exp(b_r - b_i)),  T = (I + A)^{-1}
      W  = T diag(c Gamma) K,  U = T diag(c) V,  U' = U - W S
      O  = diag(Gamma) Q S + (lower-incl-diag(Q K^T) * exp(b_r - b_i)) U'
      S <- Gamma_C S + K^T diag(Gamma_C / Gamma) U'."""
    T, dk = k.shape
    lam = np.maximum((k * k).sum(1), 1e-12)
    c = -np.expm1(-beta * lam) / lam
    S = S0.copy()
    out = np.zeros((T, v.shape[1]))
    for s in range(0, T, C):
        e = min(T, s + C)
        K, V, Q, cc = k[s:e], v[s:e], q[s:e], c[s:e]
        b = np.cumsum(log_g[s:e])
        D = np.exp(b[:, None] - b[None, :])
        n = e - s
        A = np.tril(cc[:, None] * (K @ K.T) * D, -1)
        Tm = np.zeros((n, n))
        for i in range(n):
            row = np.zeros(n)
            row[i] = 1.0
            for j in range(i):
                row -= A[i, j] * Tm[j]
            Tm[i] = row
        Gm = np.exp(b)
        W = Tm @ ((cc * Gm)[:, None] * K)
        U = Tm @ (cc[:, None] * V)
        Up = U - W @ S
        out[s:e] = Gm[:, None] * (Q @ S) + (np.tril(Q @ K.T) * np.tril(D)) @ Up
        S = Gm[-1] * S + K.T @ ((Gm[-1] / Gm)[:, None] * Up)
    return out, S


@pytest.mark.parametrize("T,C", [(32, 1), (32, 8), (37, 16), (70, 64), (64, 64)])
def test_chunked_gated_form_equals_sequential_oracle(T, C):
    d = 8
    q = RNG.standard_normal((T, d))
    k = np.stack([unit(d) * n for n in np.exp(RNG.uniform(math.log(0.1), math.log(10), T))])
    v = RNG.standard_normal((T, d))
    beta = RNG.uniform(0.05, 1.0, T)
    log_g = -RNG.uniform(0.0, 0.3, T)
    S0 = 0.3 * RNG.standard_normal((d, d))
    o, sf = oracle.fwd_gated(q[None], k[None], v[None], beta[None], log_g[None], S0[None])
    oc, sc = chunked_gated(q, k, v, beta, log_g, S0, C)
    scale = max(1.0, np.abs(o).max())
    np.testing.assert_allclose(oc, o[0], atol=1e-12 * scale)
    np.testing.assert_allclose(sc, sf[0], atol=1e-12 * scale)


def test_step_and_forward_agree():
    d = 5
    q, k, v = RNG.standard_normal(d), RNG.standard_normal(d), RNG.standard_normal(d)
    S = RNG.standard_normal((d, d))
    S1, o1 = oracle.step_gated(q, k, v, 0.6, -0.25, S)
    o, sf = oracle.fwd_gated(q[None, None], k[None, None], v[None, None], np.array([[0.6]]),
                             np.array([[-0.25]]), S[None])
    np.testing.assert_array_equal(sf[0], S1)
    np.testing.assert_array_equal(o[0, 0], o1)
