"""EFLA fp64 CPU oracle — TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. The product package never does, and
this package imports nothing from it.

The arithmetic lives in ``efla_oracle.c`` (plain C, fp64, sequential per
head); this module builds it with gcc and marshals numpy arrays through
ctypes. Every input is upcast to float64 exactly as the GPU receives it
(bf16 or fp32 values are representable in fp64 without rounding).

Method: papernotes.org note "Exact Flow Linear Attention: Exact Solution from
Continuous-Time Dynamics", section 关键设计 items 1-3 (ODE, rank-1 collapse,
exact-flow coefficient) and section 损失函数 / 训练策略 (1e-12 floor, expm1).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "efla_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

EXACT = 0
EULER = 1
RK4 = 2      # one-step RK4 of the ODE, collapsed to a scalar (rank 1)
ORDER2 = 3   # the same series cut after the second-order term

_lib = None


def build(force: bool = True) -> str:
    """Compile ``efla_oracle.c`` into ``liboracle.so`` with gcc (portable -O2,
    no -march=native so the library runs on any x86-64 host)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        cmd = ["gcc", "-std=c11", "-O2", "-fPIC", "-shared", "-o", tmp, _SRC,
               "-lm", "-lpthread"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB):
        build(force=True)
    lib = ctypes.CDLL(_LIB)
    dp = ctypes.POINTER(ctypes.c_double)
    lib.efla_oracle_alpha.restype = ctypes.c_double
    lib.efla_oracle_alpha.argtypes = [ctypes.c_double, ctypes.c_double]
    lib.efla_oracle_coef.restype = ctypes.c_double
    lib.efla_oracle_coef.argtypes = [ctypes.c_int, ctypes.c_double, ctypes.c_double]
    lib.efla_oracle_step.restype = None
    lib.efla_oracle_step.argtypes = [ctypes.c_int, dp, dp, dp, ctypes.c_double, dp, dp,
                                     ctypes.c_int, ctypes.c_int]
    lib.efla_oracle_fwd.restype = ctypes.c_int
    lib.efla_oracle_fwd.argtypes = [ctypes.c_int, dp, dp, dp, dp, dp, dp, dp, dp,
                                    ctypes.c_long, ctypes.c_long, ctypes.c_int, ctypes.c_int,
                                    ctypes.c_int]
    lib.efla_oracle_step_gated.restype = None
    lib.efla_oracle_step_gated.argtypes = [ctypes.c_int, dp, dp, dp, ctypes.c_double, ctypes.c_double,
                                           dp, dp, ctypes.c_int, ctypes.c_int]
    lib.efla_oracle_fwd_gated.restype = ctypes.c_int
    lib.efla_oracle_fwd_gated.argtypes = [ctypes.c_int, dp, dp, dp, dp, dp, dp, dp, dp,
                                          ctypes.c_long, ctypes.c_long, ctypes.c_int, ctypes.c_int,
                                          ctypes.c_int]
    lib.efla_oracle_coef_grad.restype = None
    lib.efla_oracle_coef_grad.argtypes = [ctypes.c_int, ctypes.c_double, ctypes.c_double, dp, dp]
    lib.efla_oracle_bwd.restype = ctypes.c_int
    lib.efla_oracle_bwd.argtypes = [ctypes.c_int] + [dp] * 12 + [
        ctypes.c_long, ctypes.c_long, ctypes.c_int, ctypes.c_int, ctypes.c_int]
    _lib = lib
    return lib


def _f64(x) -> np.ndarray:
    if x is None:
        return None
    if hasattr(x, "detach"):  # torch tensor: upcast exactly, on the CPU
        x = x.detach().cpu().double().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a: Optional[np.ndarray]):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def alpha(beta: float, lam: float) -> float:
    """Exact-flow coefficient (1 - e^{-beta*lam}) / lam with the 1e-12 floor."""
    return _load().efla_oracle_alpha(float(beta), float(lam))


def coef(mode: int, beta: float, lam: float) -> float:
    return _load().efla_oracle_coef(int(mode), float(beta), float(lam))


def step(q, k, v, beta: float, S, mode: int = EXACT):
    """One token on one head. Returns (S_new [dk,dv], o [dv]); inputs untouched."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    S = _f64(S).copy()
    dk, dv = S.shape
    assert q.shape == (dk,) and k.shape == (dk,) and v.shape == (dv,)
    o = np.zeros(dv, dtype=np.float64)
    _load().efla_oracle_step(int(mode), _ptr(q), _ptr(k), _ptr(v), float(beta), _ptr(S),
                             _ptr(o), dk, dv)
    return S, o


def fwd(q, k, v, beta, s0=None, mode: int = EXACT, nthreads: int = 1,
        want_norms: bool = False):
    """Sequential fp64 forward.

    q, k: [..., T, dk]; v: [..., T, dv]; beta: [..., T]; s0: [..., dk, dv] or None.
    Leading dims are flattened into independent heads. Returns (o, s_final) as
    float64 arrays of shapes [..., T, dv] and [..., dk, dv], plus the per-step
    state Frobenius norms [..., T] when ``want_norms``.
    """
    q, k, v, beta = _f64(q), _f64(k), _f64(v), _f64(beta)
    lead = beta.shape[:-1]
    T = beta.shape[-1]
    dk = k.shape[-1]
    dv = v.shape[-1]
    nh = int(np.prod(lead)) if len(lead) else 1
    assert q.shape == lead + (T, dk) and k.shape == lead + (T, dk)
    assert v.shape == lead + (T, dv)
    s0a = None
    if s0 is not None:
        s0a = _f64(s0)
        assert s0a.shape == lead + (dk, dv)
    o = np.zeros(lead + (T, dv), dtype=np.float64)
    sf = np.zeros(lead + (dk, dv), dtype=np.float64)
    sn = np.zeros(lead + (T,), dtype=np.float64) if want_norms else None
    rc = _load().efla_oracle_fwd(int(mode), _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(s0a),
                                 _ptr(o), _ptr(sf), _ptr(sn), nh, T, dk, dv, int(nthreads))
    if rc != 0:
        raise ValueError("efla_oracle_fwd rejected the sizes")
    if want_norms:
        return o, sf, sn
    return o, sf


def step_gated(q, k, v, beta: float, log_g: float, S, mode: int = EXACT):
    """One gated token on one head: S_new = exp(log_g) (I - c k k^T) S + c k v^T.
    Returns (S_new, o); inputs untouched."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    S = _f64(S).copy()
    dk, dv = S.shape
    o = np.zeros(dv, dtype=np.float64)
    _load().efla_oracle_step_gated(int(mode), _ptr(q), _ptr(k), _ptr(v), float(beta), float(log_g),
                                   _ptr(S), _ptr(o), dk, dv)
    return S, o


def fwd_gated(q, k, v, beta, log_g, s0=None, mode: int = EXACT, nthreads: int = 1):
    """Sequential fp64 forward of the gated variant: per token
    S_t = g_t (I - c_t k_t k_t^T) S_{t-1} + c_t k_t v_t^T, g_t = exp(log_g_t),
    o_t = S_t^T q_t. Shapes as fwd, log_g like beta. Returns (o, s_final)."""
    q, k, v, beta, log_g = _f64(q), _f64(k), _f64(v), _f64(beta), _f64(log_g)
    lead = beta.shape[:-1]
    T = beta.shape[-1]
    dk = k.shape[-1]
    dv = v.shape[-1]
    nh = int(np.prod(lead)) if len(lead) else 1
    assert q.shape == lead + (T, dk) and k.shape == lead + (T, dk)
    assert v.shape == lead + (T, dv) and log_g.shape == beta.shape
    s0a = None
    if s0 is not None:
        s0a = _f64(s0)
        assert s0a.shape == lead + (dk, dv)
    o = np.zeros(lead + (T, dv), dtype=np.float64)
    sf = np.zeros(lead + (dk, dv), dtype=np.float64)
    rc = _load().efla_oracle_fwd_gated(int(mode), _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(log_g),
                                       _ptr(s0a), _ptr(o), _ptr(sf), nh, T, dk, dv, int(nthreads))
    if rc != 0:
        raise ValueError("efla_oracle_fwd_gated rejected the sizes")
    return o, sf


def coef_grad(mode: int, beta: float, lam: float):
    """(dc/dbeta, dc/dlambda) of the step scalar."""
    gb, gl = ctypes.c_double(), ctypes.c_double()
    _load().efla_oracle_coef_grad(int(mode), float(beta), float(lam), ctypes.byref(gb),
                                  ctypes.byref(gl))
    return gb.value, gl.value


def bwd(q, k, v, beta, dout, s0=None, dsT=None, mode: int = EXACT, nthreads: int = 1):
    """Reverse-mode gradients of L(o, S_T) through the sequential fp64 forward.

    q, k: [..., T, dk]; v, dout: [..., T, dv]; beta: [..., T]; s0, dsT:
    [..., dk, dv] or None (zeros). Returns (dq, dk, dv, dbeta, ds0) as float64
    arrays (ds0 has the shape of one state per head)."""
    q, k, v, beta, dout = _f64(q), _f64(k), _f64(v), _f64(beta), _f64(dout)
    lead = beta.shape[:-1]
    T = beta.shape[-1]
    dk_ = k.shape[-1]
    dv_ = v.shape[-1]
    nh = int(np.prod(lead)) if len(lead) else 1
    assert q.shape == lead + (T, dk_) and k.shape == lead + (T, dk_)
    assert v.shape == lead + (T, dv_) and dout.shape == lead + (T, dv_)
    s0a = None if s0 is None else _f64(s0)
    dsa = None if dsT is None else _f64(dsT)
    for x in (s0a, dsa):
        assert x is None or x.shape == lead + (dk_, dv_)
    dq = np.zeros(lead + (T, dk_))
    dkk = np.zeros(lead + (T, dk_))
    dvv = np.zeros(lead + (T, dv_))
    db = np.zeros(lead + (T,))
    ds0 = np.zeros(lead + (dk_, dv_))
    rc = _load().efla_oracle_bwd(int(mode), _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(s0a),
                                 _ptr(dout), _ptr(dsa), _ptr(dq), _ptr(dkk), _ptr(dvv), _ptr(db),
                                 _ptr(ds0), nh, T, dk_, dv_, int(nthreads))
    if rc != 0:
        raise ValueError("efla_oracle_bwd rejected the sizes")
    return dq, dkk, dvv, db, ds0
