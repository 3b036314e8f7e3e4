"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Each test compares the oracle with something other than its own formula:
values printed on the page, scipy's matrix exponential, a fine-step RK4
integration of the ODE, a hand-written Taylor series with scaling and
squaring, mpmath at 50 digits, limits, bounds, invariants, a closed form for
orthogonal keys, and an independent chunked (WY/UT) evaluation.

Source: papernotes.org note "Exact Flow Linear Attention: Exact Solution from
Continuous-Time Dynamics" — 关键设计 item 1 (ODE dS/dt = -A S + b with
A = k k^T, b = k v^T, zero-order hold over [0, beta]), item 2 (rank-1 collapse
of exp(-beta A) and of the input integral), item 3 (contraction, alpha ->
beta - beta^2 lambda / 2), 一个完整示例 (worked example), 损失函数 / 训练策略
(1e-12 floor, expm1); the flowchart in 整体框架 (o_t = S_t^T q_t).
"""
import json
import math
import os

import mpmath
import numpy as np
import pytest
import scipy.linalg

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
RNG = np.random.default_rng(20260512)


# ----------------------------------------------------------------- helpers
def augmented_exact_update(S, k, v, beta):
    """Exact solution of dS/dt = -k k^T S + k v^T over [0, beta] with the
    inputs held constant (zero-order hold), via the augmented linear system
    d/dt [S; I] = [[-A, b], [0, 0]] [S; I] and scipy's expm (Pade, scaling
    and squaring)."""
    dk, dv = S.shape
    M = np.zeros((dk + dv, dk + dv))
    M[:dk, :dk] = -np.outer(k, k)
    M[:dk, dk:] = np.outer(k, v)
    Z0 = np.vstack([S, np.eye(dv)])
    return (scipy.linalg.expm(beta * M) @ Z0)[:dk]


def rk4_update(S, k, v, beta, hl=0.005, min_steps=400):
    """Classical RK4 on dS/dt = -k k^T S + k v^T over [0, beta], step h with
    h * lambda <= hl and at least ``min_steps`` steps."""
    lam = float(k @ k)
    n = max(min_steps, int(math.ceil(beta * lam / hl)))
    h = beta / n
    A = np.outer(k, k)
    b = np.outer(k, v)
    f = lambda X: -A @ X + b
    X = S.copy()
    for _ in range(n):
        k1 = f(X)
        k2 = f(X + 0.5 * h * k1)
        k3 = f(X + 0.5 * h * k2)
        k4 = f(X + h * k3)
        X = X + (h / 6.0) * (k1 + 2 * k2 + 2 * k3 + k4)
    return X


def taylor_expm(M, terms=30):
    """exp(M) by a truncated Taylor series with scaling and squaring."""
    nrm = np.abs(M).sum(axis=1).max()
    s = 0
    while nrm / (2 ** s) > 0.5:
        s += 1
    X = M / (2 ** s)
    E = np.eye(M.shape[0])
    term = np.eye(M.shape[0])
    for n in range(1, terms):
        term = term @ X / n
        E = E + term
    for _ in range(s):
        E = E @ E
    return E


def mp_alpha(beta, lam):
    mpmath.mp.dps = 50
    b, l = mpmath.mpf(beta), mpmath.mpf(lam)
    return float((1 - mpmath.exp(-b * l)) / l)


def transition(k, beta):
    """The oracle's homogeneous transition: one step from S = I with v = 0."""
    d = k.shape[0]
    S, _ = oracle.step(np.zeros(d), k, np.zeros(d), beta, np.eye(d))
    return S


def rand_key(d, norm):
    g = RNG.standard_normal(d)
    return g / np.linalg.norm(g) * norm


# ----------------------------------------------------------- worked example
def test_worked_example_printed_values():
    g = json.load(open(os.path.join(HERE, "golden", "worked_example.json")))
    k = np.array(g["k"])
    v = np.array(g["v"])
    S0 = np.array(g["S_prev"])
    beta = g["beta"]
    pr = g["printed"]
    tol = g["printed_precision"]

    assert float(k @ k) == pr["lambda"]
    a = oracle.alpha(beta, float(k @ k))
    assert abs(a - pr["alpha"]) <= tol
    # exact operator and its key-aligned contraction factor
    Top = transition(k, beta)
    np.testing.assert_allclose(Top, np.array(pr["exact_operator"]), atol=tol)
    assert abs(Top[0, 0] - pr["exp_minus_beta_lambda"]) <= tol
    # Euler operator (delta rule): I - beta k k^T = diag(-1, 1)
    Te, _ = oracle.step(np.zeros(2), k, np.zeros(2), beta, np.eye(2), mode=oracle.EULER)
    np.testing.assert_allclose(Te, np.array(pr["euler_operator"]), atol=1e-15)
    # full update; the page's 0.4324 is 2 x (rounded alpha), the exact 2*alpha is 0.432332
    S, _ = oracle.step(np.zeros(2), k, v, beta, S0)
    exp_S = np.array(pr["S_t"])
    assert abs(S[0, 0] - exp_S[0, 0]) <= tol
    assert abs(S[0, 1] - exp_S[0, 1]) <= 2 * tol
    assert S[1, 0] == exp_S[1, 0] and S[1, 1] == exp_S[1, 1]
    # and at full precision against the ODE's exact solution
    np.testing.assert_allclose(S, augmented_exact_update(S0, k, v, beta), atol=1e-14)


# ------------------------------------------------ closed forms / library pins
@pytest.mark.parametrize("d", [2, 3, 5, 8])
@pytest.mark.parametrize("norm", [0.1, 1.0, 4.0, 30.0])
def test_transition_equals_matrix_exponential(d, norm):
    for beta in (0.05, 0.5, 1.0):
        k = rand_key(d, norm)
        T = transition(k, beta)
        E1 = scipy.linalg.expm(-beta * np.outer(k, k))
        E2 = taylor_expm(-beta * np.outer(k, k))
        np.testing.assert_allclose(T, E1, atol=1e-12, rtol=0)
        np.testing.assert_allclose(T, E2, atol=1e-12, rtol=0)


@pytest.mark.parametrize("dk,dv", [(2, 2), (3, 5), (6, 4), (8, 8)])
def test_update_equals_exact_ode_solution(dk, dv):
    for norm in (0.2, 1.0, 3.0, 12.0):
        k = rand_key(dk, norm)
        v = RNG.standard_normal(dv)
        S = RNG.standard_normal((dk, dv))
        beta = float(RNG.uniform(0.05, 1.0))
        Sn, _ = oracle.step(np.zeros(dk), k, v, beta, S)
        ref = augmented_exact_update(S, k, v, beta)
        np.testing.assert_allclose(Sn, ref, atol=1e-12 * max(1.0, np.abs(ref).max()), rtol=0)


@pytest.mark.parametrize("norm", [0.5, 2.0, 3.7])
def test_update_equals_fine_step_rk4(norm):
    dk, dv = 4, 3
    k = rand_key(dk, norm)
    v = RNG.standard_normal(dv)
    S = RNG.standard_normal((dk, dv))
    beta = 0.8
    Sn, _ = oracle.step(np.zeros(dk), k, v, beta, S)
    ref = rk4_update(S, k, v, beta)
    assert np.abs(Sn - ref).max() <= 1e-10 * max(1.0, np.abs(ref).max())


def test_forward_sequence_equals_stepwise_ode_solution():
    """Several tokens: state by exact ODE solves, output read after each update,
    o_t = S_t^T q_t. A non-symmetric S0 and dk != dv catch transposed operands."""
    dk, dv, T = 3, 4, 7
    q = RNG.standard_normal((T, dk))
    k = np.stack([rand_key(dk, n) for n in RNG.uniform(0.3, 4.0, T)])
    v = RNG.standard_normal((T, dv))
    beta = RNG.uniform(0.1, 1.0, T)
    S0 = RNG.standard_normal((dk, dv))
    o, sf = oracle.fwd(q[None], k[None], v[None], beta[None], S0[None])
    S = S0.copy()
    for t in range(T):
        S = augmented_exact_update(S, k[t], v[t], beta[t])
        np.testing.assert_allclose(o[0, t], S.T @ q[t], atol=1e-12)
    np.testing.assert_allclose(sf[0], S, atol=1e-12)


# --------------------------------------------------------------- coefficient
def test_alpha_full_precision_mpmath():
    for beta in (0.3, 1.0):
        for x in np.logspace(-12, 3, 61):
            lam = x / beta
            a = oracle.alpha(beta, lam)
            ref = mp_alpha(beta, lam)
            assert abs(a - ref) <= 4e-16 * abs(ref), (beta, x, a, ref)


def test_alpha_small_x_limit_and_second_order_term():
    beta = 0.7
    for x in np.logspace(-9, 0, 40):
        lam = x / beta
        a = oracle.alpha(beta, lam)
        assert abs(a / beta - 1.0) <= x  # -> 1 as x -> 0
        # alternating series: |alpha - (beta - beta^2 lam / 2)| <= beta x^2 / 6,
        # plus a few fp64 ulps of beta for the rounding of both sides
        assert abs(a - (beta - 0.5 * beta * beta * lam)) <= beta * x * x / 6 + 4e-16 * beta


def test_alpha_below_beta_and_saturation():
    beta = 0.9
    for x in np.logspace(-12, 3, 91):
        lam = x / beta
        a = oracle.alpha(beta, lam)
        assert 0.0 < a < beta
        assert 0.0 < a * lam < 1.0 or (x > 36 and a * lam == 1.0)
    # stiff end: e^{-900} underflows, alpha is exactly 1/lambda, no NaN
    lam = 900.0 / beta
    assert oracle.alpha(beta, lam) == 1.0 / lam


def test_alpha_floor_on_lambda():
    # lambda = 0 is floored to 1e-12: alpha = -expm1(-beta e-12)/e-12 ~ beta
    for beta in (0.1, 0.5, 1.0):
        a = oracle.alpha(beta, 0.0)
        assert abs(a - mp_alpha(beta, 1e-12)) <= 1e-16
        assert abs(a - beta) <= beta * beta * 1e-12
    # a zero key writes nothing, whatever alpha is
    S = RNG.standard_normal((4, 4))
    Sn, o = oracle.step(np.ones(4), np.zeros(4), np.ones(4), 0.8, S)
    np.testing.assert_array_equal(Sn, S)


# ---------------------------------------------------------------- invariants
@pytest.mark.parametrize("norm", [0.3, 1.0, 5.0, 30.0])
def test_contraction_along_key(norm):
    d, beta = 6, 0.6
    k = rand_key(d, norm)
    T = transition(k, beta)
    lam = norm * norm
    ev = np.sort(np.linalg.eigvalsh(0.5 * (T + T.T)))
    ref = np.sort(np.r_[math.exp(-beta * lam), np.ones(d - 1)])
    np.testing.assert_allclose(ev, ref, atol=1e-14)
    np.testing.assert_allclose(T @ k, math.exp(-beta * lam) * k, atol=1e-13 * norm)
    for _ in range(5):
        S = RNG.standard_normal((d, 3))
        assert np.linalg.norm(T @ S) <= np.linalg.norm(S) * (1 + 1e-15)


@pytest.mark.parametrize("norm", [0.5, 2.0, 30.0])
def test_readout_along_key_blends_old_and_new(norm):
    """S_t^T k_t = e^{-beta lam} S_{t-1}^T k_t + (1 - e^{-beta lam}) v_t; with
    q = k the oracle's output is exactly that readout."""
    d, beta = 5, 1.0
    k = rand_key(d, norm)
    v = RNG.standard_normal(d)
    S = RNG.standard_normal((d, d))
    _, o = oracle.step(k, k, v, beta, S)
    e = math.exp(-beta * norm * norm)
    np.testing.assert_allclose(o, e * (S.T @ k) + (1 - e) * v,
                               atol=1e-12 * max(1, np.abs(S.T @ k).max()))


def test_orthogonal_keys_closed_form():
    """Mutually orthogonal keys commute: S_T = (I - sum a_i k_i k_i^T) S0 + sum a_i k_i v_i^T."""
    d, dv = 6, 3
    Qm, _ = np.linalg.qr(RNG.standard_normal((d, d)))
    norms = RNG.uniform(0.2, 6.0, d)
    keys = Qm.T * norms[:, None]
    betas = RNG.uniform(0.1, 1.0, d)
    vs = RNG.standard_normal((d, dv))
    S0 = RNG.standard_normal((d, dv))
    order = RNG.permutation(d)
    o, sf = oracle.fwd(np.zeros((1, d, d)), keys[order][None], vs[order][None],
                       betas[order][None], S0[None])
    P = np.eye(d)
    R = np.zeros((d, dv))
    for i in range(d):
        a = mp_alpha(betas[i], norms[i] ** 2)
        P -= a * np.outer(keys[i], keys[i])
        R += a * np.outer(keys[i], vs[i])
    np.testing.assert_allclose(sf[0], P @ S0 + R, atol=1e-13)


def test_zero_step_size_leaves_state():
    d, T = 4, 9
    q = RNG.standard_normal((1, T, d))
    k = RNG.standard_normal((1, T, d))
    v = RNG.standard_normal((1, T, d))
    S0 = RNG.standard_normal((1, d, d))
    o, sf = oracle.fwd(q, k, v, np.zeros((1, T)), S0)
    np.testing.assert_array_equal(sf, S0)
    np.testing.assert_allclose(o[0], q[0] @ S0[0], atol=1e-14)


def test_chaining_and_linearity():
    d, T, T1 = 5, 23, 9
    q = RNG.standard_normal((2, T, d))
    k = RNG.standard_normal((2, T, d))
    beta = RNG.uniform(0, 1, (2, T))
    va = RNG.standard_normal((2, T, d))
    vb = RNG.standard_normal((2, T, d))
    Sa = RNG.standard_normal((2, d, d))
    Sb = RNG.standard_normal((2, d, d))
    o, sf = oracle.fwd(q, k, va, beta, Sa)
    o1, s1 = oracle.fwd(q[:, :T1], k[:, :T1], va[:, :T1], beta[:, :T1], Sa)
    o2, s2 = oracle.fwd(q[:, T1:], k[:, T1:], va[:, T1:], beta[:, T1:], s1)
    np.testing.assert_allclose(np.concatenate([o1, o2], 1), o, atol=1e-12)
    np.testing.assert_allclose(s2, sf, atol=1e-12)
    # joint linearity in (S0, V) for fixed K and beta
    c = -1.7
    ob, sb = oracle.fwd(q, k, vb, beta, Sb)
    oc, sc = oracle.fwd(q, k, va + c * vb, beta, Sa + c * Sb)
    np.testing.assert_allclose(oc, o + c * ob, atol=1e-11)
    np.testing.assert_allclose(sc, sf + c * sb, atol=1e-11)


def test_threads_and_head_independence():
    nh, T, d = 7, 40, 6
    q = RNG.standard_normal((nh, T, d))
    k = RNG.standard_normal((nh, T, d))
    v = RNG.standard_normal((nh, T, d))
    beta = RNG.uniform(0, 1, (nh, T))
    o1, s1 = oracle.fwd(q, k, v, beta, nthreads=1)
    o4, s4 = oracle.fwd(q, k, v, beta, nthreads=4)
    np.testing.assert_array_equal(o1, o4)
    np.testing.assert_array_equal(s1, s4)
    o3, s3 = oracle.fwd(q[3:4], k[3:4], v[3:4], beta[3:4])
    np.testing.assert_array_equal(o3[0], o1[3])


def test_stiff_keys_stay_bounded_where_euler_diverges():
    """High-energy keys (beta*lambda up to ~900): the exact flow stays finite and
    bounded; the Euler (delta-rule) step on the same inputs blows up."""
    d, T = 16, 200
    k = np.stack([rand_key(d, n) for n in np.exp(RNG.uniform(0, math.log(30), T))])
    v = RNG.standard_normal((T, d))
    q = RNG.standard_normal((T, d))
    beta = 1.0 / (1.0 + np.exp(-(1.0 + RNG.standard_normal(T))))
    o, sf, sn = oracle.fwd(q[None], k[None], v[None], beta[None], want_norms=True)
    assert np.isfinite(o).all() and np.isfinite(sf).all()
    assert sn.max() < 10 * math.sqrt(d * T)
    _, _, sne = oracle.fwd(q[None], k[None], v[None], beta[None], mode=oracle.EULER,
                           want_norms=True)
    assert not np.isfinite(sne[0, -1]) or sne.max() > 1e20


# ------------------------------------------------ chunked (WY/UT) evaluation
def chunked_wy_ut(q, k, v, beta, S0, C):
    """The chunkwise-parallel form that the pages say carries over from DeltaNet
    (整体框架 and 亮点 sections): per chunk of C tokens,
      A = strictly-lower(diag(a) K K^T), T = (I + A)^{-1} by forward substitution,
      W = T diag(a) K, U = T diag(a) V, U' = U - W S,
      O = Q S + lower-incl-diag(Q K^T) U', S <- S + K^T U'.
    Written independently of the oracle (numpy, fp64); the tail chunk is ragged."""
    T, dk = k.shape
    dv = v.shape[1]
    lam = np.maximum((k * k).sum(1), 1e-12)
    a = -np.expm1(-beta * lam) / lam
    S = S0.copy()
    out = np.zeros((T, dv))
    for s in range(0, T, C):
        e = min(T, s + C)
        K, V, Q, al = k[s:e], v[s:e], q[s:e], a[s:e]
        n = e - s
        A = np.tril(al[:, None] * (K @ K.T), -1)
        Tm = np.zeros((n, n))
        for i in range(n):
            row = np.zeros(n)
            row[i] = 1.0
            for j in range(i):
                row -= A[i, j] * Tm[j]
            Tm[i] = row
        W = Tm @ (al[:, None] * K)
        U = Tm @ (al[:, None] * V)
        Up = U - W @ S
        out[s:e] = Q @ S + np.tril(Q @ K.T) @ Up
        S = S + K.T @ Up
    return out, S


@pytest.mark.parametrize("T,C", [(32, 1), (32, 4), (32, 8), (32, 32), (37, 8), (37, 16),
                                 (37, 37), (70, 64)])
def test_chunked_form_equals_sequential_oracle(T, C):
    d = 8
    q = RNG.standard_normal((T, d))
    k = np.stack([rand_key(d, n) for n in np.exp(RNG.uniform(math.log(0.1), math.log(10), T))])
    v = RNG.standard_normal((T, d))
    beta = RNG.uniform(0.05, 1.0, T)
    S0 = 0.3 * RNG.standard_normal((d, d))
    o, sf = oracle.fwd(q[None], k[None], v[None], beta[None], S0[None])
    oc, sc = chunked_wy_ut(q, k, v, beta, S0, C)
    scale = max(1.0, np.abs(o).max())
    np.testing.assert_allclose(oc, o[0], atol=1e-12 * scale)
    np.testing.assert_allclose(sc, sf[0], atol=1e-12 * scale)


# ------------------------------------------------- per-step state norm output
def test_state_norm_output_matches_ode_states():
    """The per-step output ||S_t||_F (want_norms) against the Frobenius norm of
    the state after each token, with every state taken from the augmented-ODE
    solution (scipy expm, zero-order hold over [0, beta]; 关键设计 items 1-2),
    never from the oracle. Three heads with S0 of very different scales, so a
    norm taken over the wrong head is off by orders of magnitude; the keys are
    stiff enough that the norm before a token's update differs from the norm
    after it, so a norm taken before the update fails too."""
    nh, T, d = 3, 24, 5
    scales = [0.01, 1.0, 30.0]
    q = RNG.standard_normal((nh, T, d))
    v = RNG.standard_normal((nh, T, d))
    k = np.stack([[rand_key(d, n) for n in np.exp(RNG.uniform(math.log(0.5), math.log(4), T))]
                  for _ in range(nh)])
    beta = RNG.uniform(0.3, 1.0, (nh, T))
    S0 = np.stack([s * RNG.standard_normal((d, d)) for s in scales])
    _, sf, sn = oracle.fwd(q, k, v, beta, S0, want_norms=True)
    assert sn.shape == (nh, T)
    for h in range(nh):
        S = S0[h].copy()
        before, after = [], []
        for t in range(T):
            before.append(np.linalg.norm(S))
            S = augmented_exact_update(S, k[h, t], v[h, t], beta[h, t])
            after.append(np.linalg.norm(S))
        after, before = np.array(after), np.array(before)
        np.testing.assert_allclose(sn[h], after, rtol=1e-10)
        np.testing.assert_allclose(np.linalg.norm(sf[h]), after[-1], rtol=1e-10)
        # the pin tells the two readings apart on these inputs
        assert np.abs(before - after).max() > 1e-3 * after.max()


def test_state_norm_output_special_cases():
    """beta = 0 keeps ||S_t||_F = ||S0||_F at every step (no update); k = 0 too
    (the floor makes alpha = beta, and the rank-1 terms vanish); from S0 = 0 the
    first step gives ||alpha_1 k_1 v_1^T||_F = alpha_1 ||k_1|| ||v_1|| with
    alpha_1 from mpmath (关键设计 item 2)."""
    T, d = 9, 4
    q = RNG.standard_normal((1, T, d))
    k = RNG.standard_normal((1, T, d))
    v = RNG.standard_normal((1, T, d))
    S0 = RNG.standard_normal((1, d, d))
    _, _, sn = oracle.fwd(q, k, v, np.zeros((1, T)), S0, want_norms=True)
    np.testing.assert_allclose(sn[0], np.full(T, np.linalg.norm(S0)), rtol=1e-14)
    _, _, sn = oracle.fwd(q, np.zeros_like(k), v, np.ones((1, T)), S0, want_norms=True)
    np.testing.assert_allclose(sn[0], np.full(T, np.linalg.norm(S0)), rtol=1e-14)
    beta = RNG.uniform(0.2, 0.9, (1, T))
    _, _, sn = oracle.fwd(q, k, v, beta, None, want_norms=True)
    lam = float(k[0, 0] @ k[0, 0])
    a1 = float(mp_alpha(beta[0, 0], lam))
    np.testing.assert_allclose(sn[0, 0], a1 * math.sqrt(lam) * np.linalg.norm(v[0, 0]), rtol=1e-13)
