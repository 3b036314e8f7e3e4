"""Pins of the oracle's backward (gradients of a loss of o and S_T) against
things other than its own reverse-mode code: central finite differences of
the (separately pinned) forward, torch fp64 autograd through an independent
torch loop of the recurrence, and mpmath derivatives of the step scalar.

Source of the forward being differentiated: papernotes.org note "Exact Flow
Linear Attention: Exact Solution from Continuous-Time Dynamics", 关键设计 item 2
(the update), 整体框架 (read-out after the update), 损失函数 / 训练策略 (1e-12
floor); the other step scalars as in the jsqmd.com article, section 5.3.
"""
import math

import mpmath
import numpy as np
import pytest
import torch

import oracle

RNG = np.random.default_rng(777)
MODES = [oracle.EXACT, oracle.EULER, oracle.RK4, oracle.ORDER2]


def rand_case(nh, T, dk, dv, knorm=(0.3, 1.4)):
    q = RNG.standard_normal((nh, T, dk))
    g = RNG.standard_normal((nh, T, dk))
    k = g / np.linalg.norm(g, axis=-1, keepdims=True) * RNG.uniform(*knorm, (nh, T, 1))
    v = RNG.standard_normal((nh, T, dv))
    beta = RNG.uniform(0.05, 0.9, (nh, T))
    s0 = 0.4 * RNG.standard_normal((nh, dk, dv))
    wo = RNG.standard_normal((nh, T, dv))
    ws = RNG.standard_normal((nh, dk, dv))
    return q, k, v, beta, s0, wo, ws


def loss(q, k, v, beta, s0, wo, ws, mode):
    o, sT = oracle.fwd(q, k, v, beta, s0, mode=mode)
    return float((o * wo).sum() + (sT * ws).sum())


@pytest.mark.parametrize("mode", MODES)
def test_gradients_match_central_differences(mode):
    q, k, v, beta, s0, wo, ws = rand_case(1, 7, 3, 4)
    dq, dk, dv, db, ds0 = oracle.bwd(q, k, v, beta, wo, s0, ws, mode=mode)
    h = 1e-6
    args = [q, k, v, beta, s0]
    grads = [dq, dk, dv, db, ds0]
    for ai, (x, gx) in enumerate(zip(args, grads)):
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            ap, am = list(args), list(args)
            ap[ai], am[ai] = xp, xm
            fd = (loss(*ap, wo, ws, mode) - loss(*am, wo, ws, mode)) / (2 * h)
            assert abs(fd - gx[idx]) <= 1e-7 * max(1.0, abs(fd)), (ai, idx, fd, gx[idx])


def coef_torch(mode, b, lam):
    x = b * lam
    if mode == oracle.EULER:
        return b
    if mode == oracle.RK4:
        return b * (1 - x / 2 + x * x / 6 - x * x * x / 24)
    if mode == oracle.ORDER2:
        return b * (1 - x / 2)
    lc = torch.clamp_min(lam, 1e-12)
    return -torch.expm1(-b * lc) / lc


def torch_forward(q, k, v, beta, s0, mode):
    """The recurrence as a plain torch loop (fp64), for autograd."""
    nh, T, dk = q.shape
    outs = []
    S = s0
    for t in range(T):
        kt, vt, qt = k[:, t], v[:, t], q[:, t]
        lam = (kt * kt).sum(-1)
        c = coef_torch(mode, beta[:, t], lam)
        p = torch.einsum("hij,hi->hj", S, kt)
        S = S + c[:, None, None] * kt[:, :, None] * (vt - p)[:, None, :]
        outs.append(torch.einsum("hij,hi->hj", S, qt))
    return torch.stack(outs, 1), S


# the approximate steps are unstable at stiff keys: only the exact flow there
@pytest.mark.parametrize("mode,knorm", [(m, (0.3, 1.4)) for m in MODES] + [(oracle.EXACT, (1.0, 6.0))])
def test_gradients_match_torch_autograd(mode, knorm):
    q, k, v, beta, s0, wo, ws = rand_case(3, 29, 6, 5, knorm)
    k[1, 4] = 0.0  # a zero key: the floor makes the scalar constant in lambda
    dq, dk, dv, db, ds0 = oracle.bwd(q, k, v, beta, wo, s0, ws, mode=mode, nthreads=3)
    ts = [torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v, beta, s0)]
    o, sT = torch_forward(*ts, mode)
    L = (o * torch.tensor(wo)).sum() + (sT * torch.tensor(ws)).sum()
    L.backward()
    for name, mine, t in zip("q k v beta s0".split(), (dq, dk, dv, db, ds0), ts):
        ref = t.grad.numpy()
        scale = max(1.0, np.abs(ref).max())
        np.testing.assert_allclose(mine, ref, rtol=0, atol=1e-10 * scale, err_msg=name)


def test_state_gradient_alone_and_no_initial_state():
    """dS_T only (dout = 0): ds0 is the transpose-product of the transitions;
    with s0 = None the state gradient is still reported."""
    q, k, v, beta, s0, wo, ws = rand_case(2, 11, 4, 4)
    zero = np.zeros_like(wo)
    dq, dk, dv, db, ds0 = oracle.bwd(q, k, v, beta, zero, None, ws)
    assert np.abs(dq).max() == 0.0
    P = np.stack([np.eye(4)] * 2)
    for t in range(11):
        c = np.array([oracle.coef(oracle.EXACT, beta[h, t], k[h, t] @ k[h, t]) for h in range(2)])
        P = np.einsum("hij,hjk->hik", np.eye(4) - c[:, None, None] * np.einsum("hi,hj->hij", k[:, t], k[:, t]), P)
    # S_T = P S_0 + (terms without S_0), so dL/dS_0 = P^T W_s
    np.testing.assert_allclose(ds0, np.einsum("hji,hjk->hik", P, ws), rtol=0, atol=1e-12)


@pytest.mark.parametrize("mode", MODES)
def test_scalar_derivatives_against_mpmath(mode):
    mpmath.mp.dps = 40
    for beta, lam in ((0.3, 0.7), (0.9, 2.5), (1e-3, 0.2), (0.6, 1e-7)):
        def f(b, l):
            x = b * l
            if mode == oracle.EULER:
                return b
            if mode == oracle.RK4:
                return b * (1 - x / 2 + x ** 2 / 6 - x ** 3 / 24)
            if mode == oracle.ORDER2:
                return b * (1 - x / 2)
            return (1 - mpmath.exp(-x)) / l
        gb, gl = oracle.coef_grad(mode, beta, lam)
        rb = float(mpmath.diff(lambda b: f(b, mpmath.mpf(lam)), mpmath.mpf(beta)))
        rl = float(mpmath.diff(lambda l: f(mpmath.mpf(beta), l), mpmath.mpf(lam)))
        assert abs(gb - rb) <= 1e-12 * max(1.0, abs(rb))
        assert abs(gl - rl) <= 1e-10 * max(1.0, abs(rl)), (beta, lam, gl, rl)


def chunked_backward(q, k, v, beta, s0, dout, dsT, C, mode):
    """The chunk-level backward of the WY/UT form, one head, numpy fp64. Per
    chunk with start state S, D = diag(c), A = strictly-lower(D K K^T),
    T = (I + A)^{-1}, Yh = V - K S, U = T D Yh, M = lower-incl-diag(Q K^T):
    forward O = Q S + M U, S' = S + K^T U. Given dO and dS' (the gradient for
    S'):
      dU = M^T dO + K dS',  G = T^T dU,  dYh = D G  (= dV)
      dS = dS' + Q^T dO - K^T dYh
      dM = lower-incl-diag(dO U^T),  E = strictly-lower(-G U^T)
      dc = rowsum(G * Yh) + rowsum(E * (K K^T))
      dQ = dO S^T + dM K
      dK = dM^T Q + U dS'^T - dYh S^T + D E K + E^T D K (+ 2 dc c_lambda k)
    Chunk-start states come from a forward pass; chunks run last to first."""
    T_, dk = k.shape
    lam = (k * k).sum(1)
    c = np.array([oracle.coef(mode, b, l) for b, l in zip(beta, lam)])
    cg = np.array([oracle.coef_grad(mode, b, l) for b, l in zip(beta, lam)])
    starts, S = [], s0.copy()
    for s in range(0, T_, C):
        e = min(T_, s + C)
        K, V, D = k[s:e], v[s:e], np.diag(c[s:e])
        starts.append(S.copy())
        Tm = np.linalg.inv(np.eye(e - s) + np.tril(D @ K @ K.T, -1))
        S = S + K.T @ (Tm @ D @ (V - K @ S))
    dq, dkk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    dc = np.zeros(T_)
    dS = dsT.copy()
    for ci in reversed(range(len(starts))):
        s, e = ci * C, min(T_, ci * C + C)
        K, Q, V, dO, D = k[s:e], q[s:e], v[s:e], dout[s:e], np.diag(c[s:e])
        S = starts[ci]
        Gram = K @ K.T
        Tm = np.linalg.inv(np.eye(e - s) + np.tril(D @ Gram, -1))
        Yh = V - K @ S
        U = Tm @ D @ Yh
        M = np.tril(Q @ K.T)
        dU = M.T @ dO + K @ dS
        G = Tm.T @ dU
        dYh = D @ G
        dM = np.tril(dO @ U.T)
        E = np.tril(-G @ U.T, -1)
        dc[s:e] = (G * Yh).sum(1) + (E * Gram).sum(1)
        dq[s:e] = dO @ S.T + dM @ K
        dkk[s:e] = dM.T @ Q + U @ dS.T - dYh @ S.T + D @ E @ K + E.T @ D @ K
        dv[s:e] = dYh
        dS = dS + Q.T @ dO - K.T @ dYh
    dkk += 2 * (dc * cg[:, 1])[:, None] * k
    return dq, dkk, dv, dc * cg[:, 0], dS


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("T,C", [(33, 8), (40, 16), (17, 32), (64, 16)])
def test_chunk_level_backward_equals_the_oracle(mode, T, C):
    q, k, v, beta, s0, wo, ws = rand_case(1, T, 6, 5)
    ref = oracle.bwd(q, k, v, beta, wo, s0, ws, mode=mode)
    got = chunked_backward(q[0], k[0], v[0], beta[0], s0[0], wo[0], ws[0], C, mode)
    for name, g, r in zip("dq dk dv dbeta ds0".split(), got, ref):
        r = r[0]
        np.testing.assert_allclose(g, r, rtol=0, atol=1e-11 * max(1.0, np.abs(r).max()), err_msg=name)
