"""CPU oracle for the TTT-layer forward -- test infrastructure, not the product.

Only the tests, the smoke check and the CPU-baseline leg of the benchmark may
import this package.  The library path (``chunked_linear_attention_amd``)
never imports it and shares no code with it.

``ttt_oracle.c`` holds the token-by-token fp64 implementation (see its header
for the page sections it follows and the readings it takes); this module
builds it with gcc and wraps it with ctypes.  ``dense.py`` restates the same
definitions with each chunk's sum over tokens done by a numpy matmul, for
sizes where the token loop is too slow; it is pinned against the token loop.
``decode.py`` is the single-token decode step of TTT-Linear (one gradient step
per token on a carried state, optionally anchored at the chunk-start state).
``window_attention.py`` is the causal sliding-window softmax attention that
sits beside LaCT's fast weight on the same Q, K, V.  ``backward.py`` is the
reverse-mode differentiation of the causal TTT-Linear token loop.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading
from typing import Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ttt_oracle.c")
_LIB = os.path.join(_HERE, "libttt_oracle.so")
_lock = threading.Lock()
_lib = None

LOSS_DOT = 0
LOSS_MSE = 1
CAUSAL = 0
NONCAUSAL = 1
RULE_GD = 0
RULE_MOMENTUM = 1
RULE_MUON = 2


def build(force: bool = False) -> str:
    """Compile the C oracle into oracle/libttt_oracle.so (gcc, fp64, -O2, OpenMP)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-fno-fast-math", "-ffp-contract=off", "-fopenmp",
               "-fPIC", "-shared", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is None:
            build()
            lib = ctypes.CDLL(_LIB)
            dp = ctypes.POINTER(ctypes.c_double)
            i = ctypes.c_int
            lib.oracle_ttt_linear.argtypes = [dp] * 7 + [i] * 9
            lib.oracle_ttt_linear.restype = i
            lib.oracle_lact_swiglu.argtypes = [dp] * 11 + [i] * 11
            lib.oracle_lact_swiglu.restype = i
            f = ctypes.c_double
            lib.oracle_lact_swiglu_rule.argtypes = [dp] * 11 + [i] * 11 + [f, i, f] + [dp] * 3 + [i]
            lib.oracle_lact_swiglu_rule.restype = i
            lib.oracle_max_threads.argtypes = []
            lib.oracle_max_threads.restype = i
            _lib = lib
    return _lib


def _d(x) -> np.ndarray:
    return np.ascontiguousarray(x, dtype=np.float64)


def _p(x: np.ndarray):
    return x.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def ttt_linear(q, k, v, eta, w0, *, chunk: int, loss: int, order: int = CAUSAL,
               nthreads: int = 0) -> Tuple[np.ndarray, np.ndarray]:
    """TTT-Linear forward in fp64.  q [B,H,Tq,d], k/v [B,H,Tkv,d], eta [B,H,Tkv],
    w0 [B,H,d,d] (y = x W).  Returns (out [B,H,Tq,d], w_final [B,H,d,d])."""
    lib = _load()
    q, k, v, eta, w0 = _d(q), _d(k), _d(v), _d(eta), _d(w0)
    B, H, Tq, d = q.shape
    Tkv = k.shape[2]
    assert k.shape == (B, H, Tkv, d) and v.shape == k.shape
    assert eta.shape == (B, H, Tkv) and w0.shape == (B, H, d, d)
    out = np.zeros((B, H, Tq, d))
    wf = np.zeros((B, H, d, d))
    rc = lib.oracle_ttt_linear(_p(q), _p(k), _p(v), _p(eta), _p(w0), _p(out), _p(wf), B, H, Tq,
                               Tkv, d, chunk, loss, order, nthreads)
    if rc != 0:
        raise ValueError(f"oracle_ttt_linear failed with {rc}")
    return out, wf


def lact_swiglu(q, k, v, eta, w1, w2, w3, *, chunk: int, loss: int = LOSS_DOT,
                order: int = CAUSAL, rownorm: int = 1, nthreads: int = 0):
    """LaCT SwiGLU forward in fp64.  w1, w3 [B,H,hid,d]; w2 [B,H,d,hid];
    f(x) = W2 (silu(W1 x) * (W3 x)).  Returns (out, w1_final, w2_final, w3_final)."""
    lib = _load()
    q, k, v, eta = _d(q), _d(k), _d(v), _d(eta)
    w1, w2, w3 = _d(w1), _d(w2), _d(w3)
    B, H, Tq, d = q.shape
    Tkv = k.shape[2]
    hid = w1.shape[2]
    assert w1.shape == (B, H, hid, d) and w3.shape == w1.shape and w2.shape == (B, H, d, hid)
    assert k.shape == (B, H, Tkv, d) and v.shape == k.shape and eta.shape == (B, H, Tkv)
    out = np.zeros((B, H, Tq, d))
    f1, f2, f3 = np.zeros_like(w1), np.zeros_like(w2), np.zeros_like(w3)
    rc = lib.oracle_lact_swiglu(_p(q), _p(k), _p(v), _p(eta), _p(w1), _p(w2), _p(w3), _p(out),
                                _p(f1), _p(f2), _p(f3), B, H, Tq, Tkv, d, hid, chunk, loss, order,
                                rownorm, nthreads)
    if rc != 0:
        raise ValueError(f"oracle_lact_swiglu failed with {rc}")
    return out, f1, f2, f3


def lact_swiglu_rule(q, k, v, eta, w1, w2, w3, *, chunk: int, loss: int = LOSS_DOT,
                     order: int = CAUSAL, rownorm: int = 1, rule: int = RULE_GD,
                     beta: float = 0.0, ns_steps: int = 5, lr: float = 1.0, m=None,
                     nthreads: int = 0):
    """LaCT SwiGLU forward in fp64 with an update rule: RULE_GD, RULE_MOMENTUM
    (M <- beta M + G, step M) or RULE_MUON (step lr * NS_k(M), M = G when beta is
    0).  m = (m1, m2, m3) momentum buffers shaped like the weights (zeros when
    None).  Returns (out, w1_final, w2_final, w3_final, (m1, m2, m3) after)."""
    lib = _load()
    q, k, v, eta = _d(q), _d(k), _d(v), _d(eta)
    w1, w2, w3 = _d(w1), _d(w2), _d(w3)
    B, H, Tq, d = q.shape
    Tkv = k.shape[2]
    hid = w1.shape[2]
    assert w1.shape == (B, H, hid, d) and w3.shape == w1.shape and w2.shape == (B, H, d, hid)
    assert k.shape == (B, H, Tkv, d) and v.shape == k.shape and eta.shape == (B, H, Tkv)
    if m is None:
        m = (np.zeros_like(w1), np.zeros_like(w2), np.zeros_like(w3))
    m = tuple(np.array(a, dtype=np.float64) for a in m)
    out = np.zeros((B, H, Tq, d))
    f1, f2, f3 = np.zeros_like(w1), np.zeros_like(w2), np.zeros_like(w3)
    rc = lib.oracle_lact_swiglu_rule(_p(q), _p(k), _p(v), _p(eta), _p(w1), _p(w2), _p(w3),
                                     _p(out), _p(f1), _p(f2), _p(f3), B, H, Tq, Tkv, d, hid, chunk,
                                     loss, order, rownorm, rule, float(beta), ns_steps, float(lr),
                                     _p(m[0]), _p(m[1]), _p(m[2]), nthreads)
    if rc != 0:
        raise ValueError(f"oracle_lact_swiglu_rule failed with {rc}")
    return out, f1, f2, f3, m
