"""CPU oracle for causal scaled dot-product self-attention (float64).

TEST INFRASTRUCTURE ONLY: only `tests/`, `__graft_entry__.smoke()` and the
bench's `cpu_baseline` leg may import this package.  The GPU library never
loads it and shares no code with it.

`attention_forward` / `attention_backward` wrap the plain C++ implementation in
`gattn_ref.cpp` (built by `oracle/build.py` with g++ into
`oracle/libgattn_ref.so`).  Each follows the "Let's build GPT" summary page:
tril mask with -inf above the diagonal (48:54, 55:20), row softmax (51:04),
query.key affinities (1:06:16) divided by sqrt(head size) (1:17:18), weighted
sum of values (1:10:15), heads independent (1:22:27).  The backward is the
chain rule of that forward (the pages only say the model is trained with
backprop); see the header of `gattn_ref.cpp` for the formulas.

`oracle.dropout` adds attention dropout (float64 numpy, the mask drawn with
the Philox generator of `oracle.philox`).  `oracle.rows` evaluates single
query rows and key columns (float64 numpy) for sequences too long for the
whole-problem oracle.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libgattn_ref.so")
_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _build
        _build.build()
    lib = ctypes.CDLL(_LIB_PATH)
    dp = ctypes.POINTER(ctypes.c_double)
    i = ctypes.c_int
    lib.gattn_ref_fwd.argtypes = [dp, dp, dp, dp, dp, i, i, i, i, ctypes.c_double, i]
    lib.gattn_ref_fwd.restype = None
    lib.gattn_ref_bwd.argtypes = [dp, dp, dp, dp, dp, dp, dp, dp, dp, i, i, i, i, ctypes.c_double, i]
    lib.gattn_ref_bwd.restype = None
    lib.gattn_ref_fwd_kv.argtypes = [dp, dp, dp, dp, dp, i, i, i, i, i, ctypes.c_double, i]
    lib.gattn_ref_fwd_kv.restype = None
    lib.gattn_ref_hardware_threads.argtypes = []
    lib.gattn_ref_hardware_threads.restype = i
    _lib = lib
    return lib


def _f64(x) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def hardware_threads() -> int:
    return int(_load().gattn_ref_hardware_threads())


def attention_forward(q, k, v, scale: float, nthreads: int = 0):
    """Returns (o, lse) in float64 for (B, H, T, hs) inputs."""
    lib = _load()
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, T, hs = q.shape
    assert k.shape == q.shape and v.shape == q.shape
    o = np.empty_like(q)
    lse = np.empty((B, H, T), dtype=np.float64)
    lib.gattn_ref_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, T, hs, float(scale),
                      int(nthreads))
    return o, lse


def attention_forward_kv(q, k, v, scale: float, nthreads: int = 0):
    """Forward of the newest Tq tokens: q (B, H, Tq, hs) against k, v
    (B, H, Tk, hs), Tk >= Tq; query i sees keys j <= Tk - Tq + i.  Returns
    (o, lse) in float64."""
    lib = _load()
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, Tq, hs = q.shape
    Tk = k.shape[2]
    assert k.shape == (B, H, Tk, hs) and v.shape == k.shape and Tk >= Tq
    o = np.empty_like(q)
    lse = np.empty((B, H, Tq), dtype=np.float64)
    lib.gattn_ref_fwd_kv(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, Tq, Tk, hs,
                         float(scale), int(nthreads))
    return o, lse


def attention_backward(q, k, v, dO, scale: float, nthreads: int = 0):
    """Returns (dq, dk, dv, o, lse) in float64 for (B, H, T, hs) inputs."""
    lib = _load()
    q, k, v, dO = _f64(q), _f64(k), _f64(v), _f64(dO)
    B, H, T, hs = q.shape
    assert k.shape == q.shape and v.shape == q.shape and dO.shape == q.shape
    dq, dk, dv, o = (np.empty_like(q) for _ in range(4))
    lse = np.empty((B, H, T), dtype=np.float64)
    lib.gattn_ref_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(dO), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(o),
                      _ptr(lse), B, H, T, hs, float(scale), int(nthreads))
    return dq, dk, dv, o, lse
