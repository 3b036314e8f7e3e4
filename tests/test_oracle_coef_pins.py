"""Pins of the oracle's other step coefficients (Euler, one-step RK4, second
order) against integrators of the ODE written out stage by stage, against the
matrix polynomial printed on the page, and against the exact flow in the
limit of small steps.

Sources:
- papernotes.org note "Exact Flow Linear Attention: Exact Solution from
  Continuous-Time Dynamics", 关键设计 item 1: the delta rule is one explicit
  Euler step of dS/dt = -A S + b (A = k k^T, b = k v^T) of size beta.
- jsqmd.com article "EFLA注意力机制：优化挑战与训练策略解析", section 5.3: the
  RK4 form of the step as a polynomial in A, and a second-order approximation
  named for training (read as the same series cut after the A^2 term).
"""
import math

import mpmath
import numpy as np
import pytest

import oracle

RNG = np.random.default_rng(20261203)


def rand_key(d, norm):
    g = RNG.standard_normal(d)
    return g / np.linalg.norm(g) * norm


def ode_rhs(k, v):
    A = np.outer(k, k)
    b = np.outer(k, v)
    return lambda X: -A @ X + b


def one_rk4_step(S, k, v, h):
    """One classical four-stage Runge-Kutta step of size h."""
    f = ode_rhs(k, v)
    k1 = f(S)
    k2 = f(S + 0.5 * h * k1)
    k3 = f(S + 0.5 * h * k2)
    k4 = f(S + h * k3)
    return S + (h / 6.0) * (k1 + 2 * k2 + 2 * k3 + k4)


def one_midpoint_step(S, k, v, h):
    """One explicit midpoint (second-order Runge-Kutta) step of size h."""
    f = ode_rhs(k, v)
    return S + h * f(S + 0.5 * h * f(S))


def one_euler_step(S, k, v, h):
    return S + h * ode_rhs(k, v)(S)


def printed_rk4_polynomial(S, k, v, beta):
    """The section 5.3 polynomial with explicit matrix powers of A = k k^T:
    (I - bA + b^2A^2/2 - b^3A^3/6 + b^4A^4/24) S + (bI - b^2A/2 + b^3A^2/6 - b^4A^3/24) kv^T."""
    d = k.shape[0]
    A = np.outer(k, k)
    P = [np.linalg.matrix_power(A, n) for n in range(5)]
    hom = P[0] - beta * P[1] + beta**2 * P[2] / 2 - beta**3 * P[3] / 6 + beta**4 * P[4] / 24
    inp = beta * P[0] - beta**2 * P[1] / 2 + beta**3 * P[2] / 6 - beta**4 * P[3] / 24
    assert hom.shape == (d, d)
    return hom @ S + inp @ np.outer(k, v)


def series_cut_at_second_order(S, k, v, beta):
    A = np.outer(k, k)
    I = np.eye(k.shape[0])
    return (I - beta * A + beta**2 * A @ A / 2) @ S + (beta * I - beta**2 * A / 2) @ np.outer(k, v)


CASES = [(d, n, b) for d in (2, 3, 5, 8) for n in (0.2, 1.0, 2.5) for b in (0.05, 0.5, 1.3)]


@pytest.mark.parametrize("d,norm,beta", CASES)
def test_rk4_mode_is_one_classical_rk4_step(d, norm, beta):
    k = rand_key(d, norm)
    v, q = RNG.standard_normal(d), RNG.standard_normal(d)
    S = RNG.standard_normal((d, d))
    ref = one_rk4_step(S, k, v, beta)
    got, o = oracle.step(q, k, v, beta, S, mode=oracle.RK4)
    sc = max(1.0, np.abs(ref).max())
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12 * sc)
    np.testing.assert_allclose(o, ref.T @ q, rtol=0, atol=1e-12 * sc * max(1, np.abs(q).sum()))


@pytest.mark.parametrize("d,norm,beta", CASES)
def test_rk4_mode_equals_printed_polynomial(d, norm, beta):
    k = rand_key(d, norm)
    v = RNG.standard_normal(d)
    S = RNG.standard_normal((d, d))
    ref = printed_rk4_polynomial(S, k, v, beta)
    got, _ = oracle.step(np.zeros(d), k, v, beta, S, mode=oracle.RK4)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12 * max(1.0, np.abs(ref).max()))


@pytest.mark.parametrize("d,norm,beta", CASES)
def test_order2_mode_is_one_midpoint_step_and_the_cut_series(d, norm, beta):
    k = rand_key(d, norm)
    v = RNG.standard_normal(d)
    S = RNG.standard_normal((d, d))
    got, _ = oracle.step(np.zeros(d), k, v, beta, S, mode=oracle.ORDER2)
    for ref in (one_midpoint_step(S, k, v, beta), series_cut_at_second_order(S, k, v, beta)):
        np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12 * max(1.0, np.abs(ref).max()))


@pytest.mark.parametrize("d,norm,beta", CASES)
def test_euler_mode_is_one_explicit_euler_step(d, norm, beta):
    k = rand_key(d, norm)
    v = RNG.standard_normal(d)
    S = RNG.standard_normal((d, d))
    ref = one_euler_step(S, k, v, beta)
    got, _ = oracle.step(np.zeros(d), k, v, beta, S, mode=oracle.EULER)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12 * max(1.0, np.abs(ref).max()))


def test_rk4_transition_on_the_worked_example():
    """The worked example's key and step (k = [2, 0], beta = 0.5, x = 2): RK4
    shrinks the key direction by the fourth-order Taylor value of e^{-2},
    1 - 2 + 2 - 4/3 + 2/3 = 1/3; second order by 1 - 2 + 2 = 1; Euler by -1."""
    k = np.array([2.0, 0.0])
    for mode, along in ((oracle.RK4, 1.0 / 3.0), (oracle.ORDER2, 1.0), (oracle.EULER, -1.0),
                        (oracle.EXACT, math.exp(-2.0))):
        S, _ = oracle.step(np.zeros(2), k, np.zeros(2), 0.5, np.eye(2), mode=mode)
        np.testing.assert_allclose(S, np.diag([along, 1.0]), rtol=0, atol=1e-15)


@pytest.mark.parametrize("mode,order", [(oracle.EULER, 1), (oracle.ORDER2, 2), (oracle.RK4, 4)])
def test_local_error_against_the_exact_flow_has_the_method_order(mode, order):
    """alpha - c = beta (-x)^p / (p+1)! (1 + O(x)) for a method of order p:
    the first term of the exponential series that the method drops (the exact
    alpha from mpmath at 50 digits)."""
    mpmath.mp.dps = 50
    beta, lam = 0.7, 1e-2 / 0.7  # x = 1e-2
    x = beta * lam
    alpha = (1 - mpmath.exp(-mpmath.mpf(beta) * lam)) / lam
    diff = float(alpha) - oracle.coef(mode, beta, lam)
    lead = beta * (-x) ** order / math.factorial(order + 1)
    assert abs(diff / lead - 1.0) < 2 * x


@pytest.mark.parametrize("mode", [oracle.EULER, oracle.RK4, oracle.ORDER2])
def test_sequence_equals_stepwise_integrator(mode):
    """The forward over a sequence equals one integrator step per token with
    the read-out after each step."""
    step = {oracle.EULER: one_euler_step, oracle.RK4: one_rk4_step,
            oracle.ORDER2: one_midpoint_step}[mode]
    T, dk, dv = 23, 5, 4
    q = RNG.standard_normal((T, dk))
    k = np.stack([rand_key(dk, n) for n in RNG.uniform(0.3, 1.5, T)])
    v = RNG.standard_normal((T, dv))
    beta = RNG.uniform(0.05, 0.8, T)
    S0 = 0.3 * RNG.standard_normal((dk, dv))
    o, sf = oracle.fwd(q[None], k[None], v[None], beta[None], S0[None], mode=mode)
    S = S0.copy()
    for t in range(T):
        S = step(S, k[t], v[t], beta[t])
        np.testing.assert_allclose(o[0, t], S.T @ q[t], rtol=0, atol=1e-12)
    np.testing.assert_allclose(sf[0], S, rtol=0, atol=1e-12)


def chunked_with_coefficients(q, k, v, a, S0, C):
    """The chunked WY/UT form with any per-token scalar a (its algebra uses
    only the rank-1 form of the step). numpy, fp64, ragged tail."""
    T = k.shape[0]
    S = S0.copy()
    out = np.zeros((T, v.shape[1]))
    for s in range(0, T, C):
        e = min(T, s + C)
        K, V, Q, al = k[s:e], v[s:e], q[s:e], a[s:e]
        A = np.tril(al[:, None] * (K @ K.T), -1)
        Tm = np.linalg.inv(np.eye(e - s) + A)
        Up = Tm @ (al[:, None] * (V - K @ S))
        out[s:e] = Q @ S + np.tril(Q @ K.T) @ Up
        S = S + K.T @ Up
    return out, S


@pytest.mark.parametrize("mode", [oracle.EULER, oracle.RK4, oracle.ORDER2])
@pytest.mark.parametrize("C", [4, 16])
def test_chunked_form_holds_for_every_coefficient(mode, C):
    T, d = 41, 6
    q = RNG.standard_normal((T, d))
    k = np.stack([rand_key(d, n) for n in RNG.uniform(0.2, 1.2, T)])
    v = RNG.standard_normal((T, d))
    beta = RNG.uniform(0.05, 0.9, T)
    S0 = 0.3 * RNG.standard_normal((d, d))
    a = np.array([oracle.coef(mode, b, float(kk @ kk)) for b, kk in zip(beta, k)])
    o, sf = oracle.fwd(q[None], k[None], v[None], beta[None], S0[None], mode=mode)
    oc, sc = chunked_with_coefficients(q, k, v, a, S0, C)
    scale = max(1.0, np.abs(o).max())
    np.testing.assert_allclose(oc, o[0], rtol=0, atol=1e-11 * scale)
    np.testing.assert_allclose(sc, sf[0], rtol=0, atol=1e-11 * scale)
