"""Exact Flow Linear Attention (EFLA) forward on MI355X (gfx950).

Thin Python binding over the C ABI in ``include/efla.h`` (library
``libefla.so`` next to this file, built by ``build.py``). The functions carry
the C entry points' names and only marshal arguments: torch provides device
memory and the current HIP stream; every step of the computation runs in the
library's HIP kernels. There is no fallback: if the library is missing the
import of the binding functions raises.

Method: papernotes.org note "Exact Flow Linear Attention: Exact Solution from
Continuous-Time Dynamics" (关键设计 items 1-3; 整体框架 for the chunked WY/UT and
recurrent forms; 损失函数 / 训练策略 for the 1e-12 floor and expm1).
"""
from __future__ import annotations

import ctypes
import os
import threading
from typing import Optional, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libefla.so")

EFLA_DTYPE_F32 = 0
EFLA_DTYPE_BF16 = 1
_DTYPES = {torch.float32: EFLA_DTYPE_F32, torch.bfloat16: EFLA_DTYPE_BF16}

STATUS_NAMES = {
    0: "EFLA_OK",
    1: "EFLA_ERR_NULL_POINTER",
    2: "EFLA_ERR_BAD_SHAPE",
    3: "EFLA_ERR_UNSUPPORTED",
    4: "EFLA_ERR_MISALIGNED",
    5: "EFLA_ERR_WORKSPACE",
    6: "EFLA_ERR_HIP",
    7: "EFLA_ERR_SCRATCH_LIMIT",
}

# Step coefficient rules (efla_coef): the exact flow, explicit Euler (the
# delta rule), one classical RK4 step and the series cut at second order.
COEFS = {"exact": 0, "euler": 1, "rk4": 2, "order2": 3}

SUPPORTED_HEAD_DIMS = (16, 32, 64, 128)
SUPPORTED_CHUNKS = (16, 32, 64)


class EflaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


_lib = None
_lock = threading.Lock()


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load ``libefla.so`` and declare the C signatures. Raises if not built."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(path):
            raise RuntimeError(
                f"{path} is not built; build it with `python -c 'import __graft_entry__ as g; g.build()'`"
                " (hipcc, gfx950). There is no CPU fallback.")
        lib = ctypes.CDLL(path)
        vp, i, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
        lib.efla_fwd_chunked_workspace_bytes.restype = sz
        lib.efla_fwd_chunked_workspace_bytes.argtypes = [i, i, i, i, i, i, i]
        lib.efla_fwd_chunked.restype = i
        lib.efla_fwd_chunked.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, sz,
                                         i, i, i, i, i, i, i, i, vp]
        lib.efla_fwd_recurrent_step.restype = i
        lib.efla_fwd_recurrent_step.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, vp]
        lib.efla_bwd_chunked_workspace_bytes.restype = sz
        lib.efla_bwd_chunked_workspace_bytes.argtypes = [i, i, i, i, i, i, i]
        lib.efla_bwd_chunked.restype = i
        lib.efla_bwd_chunked.argtypes = [vp] * 13 + [sz] + [i] * 8 + [vp]
        lib.efla_bwd_chunked_saved.restype = i
        lib.efla_bwd_chunked_saved.argtypes = [vp] * 12 + [sz] + [i] * 8 + [vp]
        lib.efla_fwd_chunked_train.restype = i
        lib.efla_fwd_chunked_train.argtypes = [vp] * 8 + [sz] + [i] * 8 + [vp]
        lib.efla_fwd_chunked_noalloc.restype = i
        lib.efla_fwd_chunked_noalloc.argtypes = [vp] * 7 + [i] * 8 + [vp]
        lib.efla_fwd_chunked_gated.restype = i
        lib.efla_fwd_chunked_gated.argtypes = [vp] * 8 + [i] * 8 + [vp]
        lib.efla_fwd_recurrent_step_gated.restype = i
        lib.efla_fwd_recurrent_step_gated.argtypes = [vp] * 7 + [i] * 6 + [vp]
        lib.efla_status_string.restype = ctypes.c_char_p
        lib.efla_status_string.argtypes = [i]
        _lib = lib
        return lib


def status_string(status: int) -> str:
    return load_library().efla_status_string(int(status)).decode()


def _raise(status: int):
    if status != 0:
        raise EflaError(status, status_string(status))


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device: torch.device, stream=None):
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return ctypes.c_void_p(s.cuda_stream)


def _keep(stream, *tensors):
    """Tie the binding's own allocations (outputs, workspaces) to a launch
    stream that is not torch's current one: the caching allocator then does
    not hand their memory to later work on the current stream while the
    kernels on ``stream`` may still use it."""
    if stream is None:
        return
    for t in tensors:
        if t is not None:
            t.record_stream(stream)


def _require(t: torch.Tensor, name: str, dtype, device, shape=None):
    """Device, dtype, contiguity and (when given) the exact shape. The C ABI
    receives bare pointers and cannot see sizes, so a buffer that is too
    small is caught here or not at all."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _coef(coef) -> int:
    if isinstance(coef, str):
        if coef not in COEFS:
            raise ValueError(f"unknown coefficient rule {coef!r}; one of {sorted(COEFS)}")
        return COEFS[coef]
    return int(coef)


def efla_fwd_chunked_workspace_bytes(B: int, H: int, T: int, d_k: int, d_v: int, chunk: int,
                                     dtype: torch.dtype) -> int:
    return int(load_library().efla_fwd_chunked_workspace_bytes(B, H, T, d_k, d_v, chunk,
                                                               _DTYPES[dtype]))


def efla_fwd_chunked(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, beta: torch.Tensor,
                     s0: Optional[torch.Tensor] = None, chunk: int = 64,
                     o: Optional[torch.Tensor] = None, s_final: Optional[torch.Tensor] = None,
                     return_state: bool = True, stream=None, coef="exact"
                     ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Chunked EFLA forward. q, k: [B,H,T,d]; v: [B,H,T,d]; beta: [B,H,T]
    (all fp32 or all bf16, contiguous, on one GPU); s0: [B,H,d,d] fp32 or None.
    Returns (o [B,H,T,d] in the input dtype, S_T [B,H,d,d] fp32 or None).
    ``s_final`` may be passed (and may be ``s0`` itself to advance in place).
    ``coef`` picks the step scalar: "exact" (EFLA), "euler", "rk4", "order2"."""
    lib = load_library()
    dev = q.device
    if q.dim() != 4:
        raise ValueError("q must be [B, H, T, d]")
    B, H, T, d = q.shape
    dt = q.dtype
    if dt not in _DTYPES:
        raise ValueError(f"unsupported dtype {dt}")
    for name, t in (("q", q), ("k", k), ("v", v), ("beta", beta)):
        _require(t, name, dt, dev)
    if k.shape != q.shape or v.shape[:3] != q.shape[:3] or beta.shape != (B, H, T):
        raise ValueError("shape mismatch between q, k, v, beta")
    dv = v.shape[3]
    if s0 is not None:
        _require(s0, "s0", torch.float32, dev)
        if s0.shape != (B, H, d, dv):
            raise ValueError("s0 must be [B, H, d_k, d_v]")
    own = []
    if o is None:
        o = torch.empty((B, H, T, dv), dtype=dt, device=dev)
        own.append(o)
    else:
        _require(o, "o", dt, dev, (B, H, T, dv))
    if s_final is None and return_state:
        s_final = torch.empty((B, H, d, dv), dtype=torch.float32, device=dev)
        own.append(s_final)
    elif s_final is not None:
        _require(s_final, "s_final", torch.float32, dev, (B, H, d, dv))
    ws_bytes = int(lib.efla_fwd_chunked_workspace_bytes(B, H, T, d, dv, chunk, _DTYPES[dt]))
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev) if ws_bytes > 0 else None
    st = lib.efla_fwd_chunked(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(s0), _ptr(o),
                              _ptr(s_final), _ptr(ws), ws_bytes, B, H, T, d, dv, int(chunk),
                              _coef(coef), _DTYPES[dt], _stream(dev, stream))
    _raise(st)
    _keep(stream, ws, *own)
    return o, s_final


def efla_fwd_chunked_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, beta: torch.Tensor,
                             s0: Optional[torch.Tensor], o: torch.Tensor, s_final: Optional[torch.Tensor],
                             chunk: int = 64, stream=None, coef="exact") -> None:
    """efla_fwd_chunked through the C entry point that allocates nothing: the
    caller passes o (and s_final, or None) and the library's fixed scratch
    serves the time-segmented path. Same checks as efla_fwd_chunked; calls
    that overlap in time on one GPU must not be made."""
    lib = load_library()
    dev = q.device
    if q.dim() != 4:
        raise ValueError("q must be [B, H, T, d]")
    B, H, T, d = q.shape
    dt = q.dtype
    if dt not in _DTYPES:
        raise ValueError(f"unsupported dtype {dt}")
    for name, t in (("q", q), ("k", k), ("v", v), ("beta", beta)):
        _require(t, name, dt, dev)
    if k.shape != q.shape or v.shape != q.shape or beta.shape != (B, H, T):
        raise ValueError("shape mismatch between q, k, v, beta")
    if s0 is not None:
        _require(s0, "s0", torch.float32, dev, (B, H, d, d))
    _require(o, "o", dt, dev, (B, H, T, d))
    if s_final is not None:
        _require(s_final, "s_final", torch.float32, dev, (B, H, d, d))
    st = lib.efla_fwd_chunked_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(s0), _ptr(o),
                                      _ptr(s_final), B, H, T, d, d, int(chunk), _coef(coef),
                                      _DTYPES[dt], _stream(dev, stream))
    _raise(st)


def efla_fwd_chunked_gated(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, beta: torch.Tensor,
                           log_g: torch.Tensor, s0: Optional[torch.Tensor] = None, chunk: int = 64,
                           o: Optional[torch.Tensor] = None, s_final: Optional[torch.Tensor] = None,
                           return_state: bool = True, stream=None, coef="exact"
                           ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Gated EFLA forward: S_t = g_t (I - c_t k_t k_t^T) S_{t-1} + c_t k_t v_t^T
    with g_t = exp(log_g_t); log_g [B,H,T] fp32 (values <= 0 keep every decay
    factor at most 1; positive values are allowed). Everything else as
    efla_fwd_chunked, s_final aliasing s0 included."""
    lib = load_library()
    dev = q.device
    if q.dim() != 4:
        raise ValueError("q must be [B, H, T, d]")
    B, H, T, d = q.shape
    dt = q.dtype
    if dt not in _DTYPES:
        raise ValueError(f"unsupported dtype {dt}")
    for name, t in (("q", q), ("k", k), ("v", v), ("beta", beta)):
        _require(t, name, dt, dev)
    if k.shape != q.shape or v.shape != q.shape or beta.shape != (B, H, T):
        raise ValueError("shape mismatch between q, k, v, beta")
    _require(log_g, "log_g", torch.float32, dev, (B, H, T))
    if s0 is not None:
        _require(s0, "s0", torch.float32, dev, (B, H, d, d))
    own = []
    if o is None:
        o = torch.empty((B, H, T, d), dtype=dt, device=dev)
        own.append(o)
    else:
        _require(o, "o", dt, dev, (B, H, T, d))
    if s_final is None and return_state:
        s_final = torch.empty((B, H, d, d), dtype=torch.float32, device=dev)
        own.append(s_final)
    elif s_final is not None:
        _require(s_final, "s_final", torch.float32, dev, (B, H, d, d))
    st = lib.efla_fwd_chunked_gated(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(log_g), _ptr(s0),
                                    _ptr(o), _ptr(s_final), B, H, T, d, d, int(chunk), _coef(coef),
                                    _DTYPES[dt], _stream(dev, stream))
    _raise(st)
    _keep(stream, *own)
    return o, s_final


def efla_fwd_recurrent_step_gated(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                                  beta: torch.Tensor, log_g: torch.Tensor, state: torch.Tensor,
                                  o: Optional[torch.Tensor] = None, stream=None,
                                  coef="exact") -> torch.Tensor:
    """One gated token per head: q, k, v [B,H,d]; beta [B,H]; log_g [B,H] fp32;
    state [B,H,d,d] fp32 advanced in place. Returns o [B,H,d]."""
    lib = load_library()
    dev = q.device
    if q.dim() != 3:
        raise ValueError("q must be [B, H, d]")
    B, H, d = q.shape
    dt = q.dtype
    if dt not in _DTYPES:
        raise ValueError(f"unsupported dtype {dt}")
    for name, t in (("q", q), ("k", k), ("v", v), ("beta", beta)):
        _require(t, name, dt, dev)
    if k.shape != q.shape or v.shape != q.shape or beta.shape != (B, H):
        raise ValueError("shape mismatch between q, k, v, beta")
    _require(log_g, "log_g", torch.float32, dev, (B, H))
    _require(state, "state", torch.float32, dev, (B, H, d, d))
    own = None
    if o is None:
        o = own = torch.empty((B, H, d), dtype=dt, device=dev)
    else:
        _require(o, "o", dt, dev, (B, H, d))
    st = lib.efla_fwd_recurrent_step_gated(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(log_g),
                                           _ptr(state), _ptr(o), B, H, d, d, _coef(coef), _DTYPES[dt],
                                           _stream(dev, stream))
    _raise(st)
    _keep(stream, own)
    return o


def efla_fwd_recurrent_step(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                            beta: torch.Tensor, state: torch.Tensor,
                            o: Optional[torch.Tensor] = None, stream=None,
                            coef="exact") -> torch.Tensor:
    """One token per head: q, k, v [B,H,d]; beta [B,H]; state [B,H,d,d] fp32,
    advanced in place. Returns o [B,H,d] = S_t^T q_t in the input dtype.
    ``coef`` as in efla_fwd_chunked."""
    lib = load_library()
    dev = q.device
    if q.dim() != 3:
        raise ValueError("q must be [B, H, d]")
    B, H, d = q.shape
    dt = q.dtype
    if dt not in _DTYPES:
        raise ValueError(f"unsupported dtype {dt}")
    for name, t in (("q", q), ("k", k), ("v", v), ("beta", beta)):
        _require(t, name, dt, dev)
    if k.shape != q.shape or v.shape[:2] != (B, H) or beta.shape != (B, H):
        raise ValueError("shape mismatch between q, k, v, beta")
    dv = v.shape[2]
    _require(state, "state", torch.float32, dev)
    if state.shape != (B, H, d, dv):
        raise ValueError("state must be [B, H, d_k, d_v]")
    own = None
    if o is None:
        o = own = torch.empty((B, H, dv), dtype=dt, device=dev)
    else:
        _require(o, "o", dt, dev, (B, H, dv))
    st = lib.efla_fwd_recurrent_step(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(state),
                                     _ptr(o), B, H, d, dv, _coef(coef), _DTYPES[dt],
                                     _stream(dev, stream))
    _raise(st)
    _keep(stream, own)
    return o


def efla_bwd_chunked_workspace_bytes(B: int, H: int, T: int, d_k: int, d_v: int, chunk: int,
                                     dtype: torch.dtype) -> int:
    return int(load_library().efla_bwd_chunked_workspace_bytes(B, H, T, d_k, d_v, chunk,
                                                               _DTYPES[dtype]))


def efla_fwd_chunked_train(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, beta: torch.Tensor,
                           s0: Optional[torch.Tensor] = None, chunk: int = 64, coef="exact",
                           o: Optional[torch.Tensor] = None, s_final: Optional[torch.Tensor] = None,
                           stream=None):
    """Forward of a training step: the outputs of efla_fwd_chunked plus the
    chunk-start states, kept for the backward. Returns (o, s_final, saved),
    where ``saved`` is the backward workspace to pass to
    ``efla_bwd_chunked(..., saved_workspace=saved)``."""
    lib = load_library()
    dev = q.device
    if q.dim() != 4:
        raise ValueError("q must be [B, H, T, d]")
    B, H, T, d = q.shape
    dt = q.dtype
    if dt not in _DTYPES:
        raise ValueError(f"unsupported dtype {dt}")
    for name, t in (("q", q), ("k", k), ("v", v), ("beta", beta)):
        _require(t, name, dt, dev)
    if k.shape != q.shape or v.shape != q.shape or beta.shape != (B, H, T):
        raise ValueError("shape mismatch between q, k, v, beta")
    if s0 is not None:
        _require(s0, "s0", torch.float32, dev)
        if s0.shape != (B, H, d, d):
            raise ValueError("s0 must be [B, H, d_k, d_v]")
    own = []
    if o is None:
        o = torch.empty_like(q)
        own.append(o)
    else:
        _require(o, "o", dt, dev, (B, H, T, d))
    if s_final is None:
        s_final = torch.empty((B, H, d, d), dtype=torch.float32, device=dev)
        own.append(s_final)
    else:
        _require(s_final, "s_final", torch.float32, dev, (B, H, d, d))
    ws_bytes = int(lib.efla_bwd_chunked_workspace_bytes(B, H, T, d, d, chunk, _DTYPES[dt]))
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
    st = lib.efla_fwd_chunked_train(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(s0), _ptr(o),
                                    _ptr(s_final), _ptr(ws), ws_bytes, B, H, T, d, d, int(chunk),
                                    _coef(coef), _DTYPES[dt], _stream(dev, stream))
    _raise(st)
    _keep(stream, ws, *own)
    return o, s_final, ws


def efla_bwd_chunked(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, beta: torch.Tensor,
                     dout: torch.Tensor, s0: Optional[torch.Tensor] = None,
                     ds_final: Optional[torch.Tensor] = None, chunk: int = 64, coef="exact",
                     want_ds0: bool = True, stream=None,
                     saved_workspace: Optional[torch.Tensor] = None):
    """Backward of efla_fwd_chunked for a loss L(o, S_T): given dout = dL/do
    [B,H,T,d] (input dtype) and ds_final = dL/dS_T [B,H,d,d] fp32 or None,
    returns (dq, dk, dv, dbeta, ds0) with dq, dk, dv, dbeta in the input dtype
    and ds0 fp32 (None unless want_ds0). With ``saved_workspace`` (the third
    result of efla_fwd_chunked_train for the same inputs) the forward is not
    recomputed."""
    lib = load_library()
    dev = q.device
    if q.dim() != 4:
        raise ValueError("q must be [B, H, T, d]")
    B, H, T, d = q.shape
    dt = q.dtype
    if dt not in _DTYPES:
        raise ValueError(f"unsupported dtype {dt}")
    for name, t in (("q", q), ("k", k), ("v", v), ("beta", beta), ("dout", dout)):
        _require(t, name, dt, dev)
    if k.shape != q.shape or v.shape != q.shape or dout.shape != q.shape or beta.shape != (B, H, T):
        raise ValueError("shape mismatch between q, k, v, beta, dout")
    for name, t in (("s0", s0), ("ds_final", ds_final)):
        if t is not None:
            _require(t, name, torch.float32, dev)
            if t.shape != (B, H, d, d):
                raise ValueError(f"{name} must be [B, H, d_k, d_v]")
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    db = torch.empty_like(beta)
    ds0 = torch.empty((B, H, d, d), dtype=torch.float32, device=dev) if want_ds0 else None
    ws_bytes = int(lib.efla_bwd_chunked_workspace_bytes(B, H, T, d, d, chunk, _DTYPES[dt]))
    if saved_workspace is not None:
        _require(saved_workspace, "saved_workspace", torch.uint8, dev)
        if saved_workspace.numel() < ws_bytes:
            raise ValueError("saved_workspace is smaller than the backward workspace for these sizes")
        st = lib.efla_bwd_chunked_saved(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(dout),
                                        _ptr(ds_final), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(db),
                                        _ptr(ds0), _ptr(saved_workspace), ws_bytes, B, H, T, d, d,
                                        int(chunk), _coef(coef), _DTYPES[dt], _stream(dev, stream))
        _raise(st)
        _keep(stream, dq, dk, dv, db, ds0)
        return dq, dk, dv, db, ds0
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
    st = lib.efla_bwd_chunked(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(s0), _ptr(dout),
                              _ptr(ds_final), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(db), _ptr(ds0),
                              _ptr(ws), ws_bytes, B, H, T, d, d, int(chunk), _coef(coef),
                              _DTYPES[dt], _stream(dev, stream))
    _raise(st)
    _keep(stream, ws, dq, dk, dv, db, ds0)
    return dq, dk, dv, db, ds0
