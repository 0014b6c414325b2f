"""Seeded synthetic inputs for the TTT-layer forward (TTT-Linear and LaCT SwiGLU).

This module is the only code shared by the CPU oracle side (tests, the CPU
baseline) and the HIP side (tests, bench, smoke).  It draws random numbers and
shapes them into the value distributions of the workloads; it contains none of
the method's arithmetic (no fast-weight update, no apply, no loss).

Recipe (every workload):
  * ``numpy.random.default_rng(seed)`` (PCG64); fp64 standard normals drawn in
    the order Q, K, V, eta-noise, then the initial state (W, or W1, W2, W3),
    each in C order over its array shape.
  * Q and K rows are L2-normalised when the workload says so, otherwise scaled.
  * The learning rate is a transform of its noise (constant, 0.1*sigmoid,
    0.01*softplus).
  * Everything is cast to fp32.  For bf16 workloads Q, K and V are then rounded
    to bf16 with round-to-nearest-even; the rounded values (widened back to
    fp32) are what both the oracle and the GPU consume.  eta and the state
    stay fp32.

Layouts: q [B,H,Tq,d]; k, v [B,H,Tkv,d]; eta [B,H,Tkv];
TTT-Linear state w [B,H,d,d] (row-vector convention y = x.W, w[in][out]);
LaCT states w1, w3 [B,H,hid,d] and w2 [B,H,d,hid] (column convention
f(x) = W2 (silu(W1 x) * (W3 x))).
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional

import numpy as np

LOSS_DOT = 0
LOSS_MSE = 1
CAUSAL = 0
NONCAUSAL = 1


# ----------------------------------------------------------------------------
# bf16 helpers (round to nearest even), numpy only
# ----------------------------------------------------------------------------
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest even) and return the uint16 bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    rounding = ((u >> 16) & 1) + 0x7FFF
    out = ((u + rounding) >> 16).astype(np.uint16)
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def round_bf16(x: np.ndarray) -> np.ndarray:
    return bf16_bits_to_f32(f32_to_bf16_bits(x))


def _l2_rows(x: np.ndarray) -> np.ndarray:
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
    return x / n


# ----------------------------------------------------------------------------
# Workload definitions (the five workloads of the metric, plus free shapes)
# ----------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class LinearWorkload:
    name: str
    B: int
    H: int
    T: int
    d: int
    chunk: int
    loss: int
    dtype: str          # "f32" or "bf16"
    qk_dist: str        # "scaled" (N(0,1)/sqrt(d)) or "l2" (row-normalised)
    v_dist: str         # "scaled" or "normal"
    eta_dist: str       # "const0.1" or "sigmoid0.1"
    w0: str             # "zeros" or "identity"
    order: int = CAUSAL
    Tq: Optional[int] = None   # non-causal only


@dataclasses.dataclass(frozen=True)
class LactWorkload:
    name: str
    B: int
    H: int
    Tkv: int
    Tq: int
    d: int
    hid: int
    chunk: int
    loss: int
    order: int
    dtype: str = "bf16"
    rownorm: int = 1


# TTT-Linear, inner-product loss, fp32, 1x1 heads, T=256, d=64, b=16.
TINY_DOT = LinearWorkload("ttt_linear_dot_T256_d64_b16_f32", 1, 1, 256, 64, 16, LOSS_DOT,
                          "f32", "scaled", "scaled", "const0.1", "zeros")
# TTT-Linear, MSE loss, bf16, 4x8 heads, T=4096, d=64, b=16.
MSE_D64 = LinearWorkload("ttt_linear_mse_B4_H8_T4096_d64_b16_bf16", 4, 8, 4096, 64, 16, LOSS_MSE,
                         "bf16", "l2", "normal", "sigmoid0.1", "identity")


def mse_d128(chunk: int) -> LinearWorkload:
    """TTT-Linear, MSE loss, bf16, 2x16 heads, T=16384, d=128, chunk sweep."""
    return LinearWorkload(f"ttt_linear_mse_B2_H16_T16384_d128_b{chunk}_bf16", 2, 16, 16384, 128,
                          chunk, LOSS_MSE, "bf16", "l2", "normal", "sigmoid0.1", "identity")


# LaCT causal LM layer: d=256, hidden 512, b=2048, 4 heads, T=32768.
LACT_CAUSAL = LactWorkload("lact_swiglu_causal_H4_T32768_d256_h512_b2048", 1, 4, 32768, 32768,
                           256, 512, 2048, LOSS_DOT, CAUSAL)
# LaCT non-causal: d=384, hidden 768, 2 heads, 65536 update tokens, 16384 queries.
LACT_NONCAUSAL = LactWorkload("lact_swiglu_noncausal_H2_Tkv65536_Tq16384_d384_h768", 1, 2, 65536,
                              16384, 384, 768, 65536, LOSS_DOT, NONCAUSAL)

WORKLOAD_SEEDS = {TINY_DOT.name: 1, MSE_D64.name: 2, LACT_CAUSAL.name: 4, LACT_NONCAUSAL.name: 5}
for _b in (16, 64, 256, 1024):
    WORKLOAD_SEEDS[mse_d128(_b).name] = 3


# ----------------------------------------------------------------------------
# Generators
# ----------------------------------------------------------------------------
def gen_linear(B: int, H: int, Tq: int, Tkv: int, d: int, *, seed: int, dtype: str = "bf16",
               qk_dist: str = "l2", v_dist: str = "normal", eta_dist: str = "sigmoid0.1",
               w0: str = "identity", eta_scale: float = 1.0) -> Dict[str, np.ndarray]:
    """TTT-Linear inputs.  Returns fp32 numpy arrays q, k, v, eta, w0 (values exactly
    representable in the workload dtype) plus, for bf16, the bit patterns q16/k16/v16."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, H, Tq, d))
    k = rng.standard_normal((B, H, Tkv, d))
    v = rng.standard_normal((B, H, Tkv, d))
    e = rng.standard_normal((B, H, Tkv))
    if qk_dist == "l2":
        q, k = _l2_rows(q), _l2_rows(k)
    elif qk_dist == "scaled":
        q, k = q / np.sqrt(d), k / np.sqrt(d)
    else:
        raise ValueError(qk_dist)
    if v_dist == "scaled":
        v = v / np.sqrt(d)
    elif v_dist != "normal":
        raise ValueError(v_dist)
    if eta_dist == "const0.1":
        eta = np.full((B, H, Tkv), 0.1)
    elif eta_dist == "sigmoid0.1":
        eta = 0.1 / (1.0 + np.exp(-e))
    else:
        raise ValueError(eta_dist)
    eta = eta * eta_scale
    if w0 == "zeros":
        w = np.zeros((B, H, d, d))
    elif w0 == "identity":
        w = np.broadcast_to(np.eye(d), (B, H, d, d)).copy()
    elif w0 == "normal":
        w = rng.standard_normal((B, H, d, d)) / np.sqrt(d)
    else:
        raise ValueError(w0)
    out = {"q": q.astype(np.float32), "k": k.astype(np.float32), "v": v.astype(np.float32),
           "eta": eta.astype(np.float32), "w0": w.astype(np.float32)}
    if dtype == "bf16":
        for n in ("q", "k", "v"):
            bits = f32_to_bf16_bits(out[n])
            out[n + "16"] = bits
            out[n] = bf16_bits_to_f32(bits)
    elif dtype != "f32":
        raise ValueError(dtype)
    return out


def gen_linear_workload(wl: LinearWorkload, seed: Optional[int] = None,
                        T: Optional[int] = None) -> Dict[str, np.ndarray]:
    """Inputs of a named TTT-Linear workload; ``T`` optionally truncates the sequence
    (the first T tokens of a shorter draw with the same recipe)."""
    seed = WORKLOAD_SEEDS.get(wl.name, 0) if seed is None else seed
    T = wl.T if T is None else T
    Tq = T if wl.order == CAUSAL else (wl.Tq or T)
    return gen_linear(wl.B, wl.H, Tq, T, wl.d, seed=seed, dtype=wl.dtype, qk_dist=wl.qk_dist,
                      v_dist=wl.v_dist, eta_dist=wl.eta_dist, w0=wl.w0)


def gen_lact(B: int, H: int, Tq: int, Tkv: int, d: int, hid: int, *, seed: int,
             dtype: str = "bf16", eta_scale: float = 1.0,
             w_scale: float = 1.0) -> Dict[str, np.ndarray]:
    """LaCT SwiGLU inputs: Q/K rows L2-normalised, V ~ N(0,1), eta = 0.01*softplus(N(0,1)),
    W1, W3 ~ N(0, 1/d) [hid,d], W2 ~ N(0, 1/hid) [d,hid]."""
    rng = np.random.default_rng(seed)
    q = _l2_rows(rng.standard_normal((B, H, Tq, d)))
    k = _l2_rows(rng.standard_normal((B, H, Tkv, d)))
    v = rng.standard_normal((B, H, Tkv, d))
    e = rng.standard_normal((B, H, Tkv))
    eta = 0.01 * np.logaddexp(0.0, e) * eta_scale
    w1 = rng.standard_normal((B, H, hid, d)) / np.sqrt(d) * w_scale
    w2 = rng.standard_normal((B, H, d, hid)) / np.sqrt(hid) * w_scale
    w3 = rng.standard_normal((B, H, hid, d)) / np.sqrt(d) * w_scale
    out = {"q": q.astype(np.float32), "k": k.astype(np.float32), "v": v.astype(np.float32),
           "eta": eta.astype(np.float32), "w1": w1.astype(np.float32),
           "w2": w2.astype(np.float32), "w3": w3.astype(np.float32)}
    if dtype == "bf16":
        for n in ("q", "k", "v"):
            bits = f32_to_bf16_bits(out[n])
            out[n + "16"] = bits
            out[n] = bf16_bits_to_f32(bits)
    elif dtype != "f32":
        raise ValueError(dtype)
    return out


def gen_lact_workload(wl: LactWorkload, seed: Optional[int] = None, Tkv: Optional[int] = None,
                      Tq: Optional[int] = None) -> Dict[str, np.ndarray]:
    seed = WORKLOAD_SEEDS.get(wl.name, 0) if seed is None else seed
    Tkv = wl.Tkv if Tkv is None else Tkv
    if Tq is None:
        Tq = Tkv if wl.order == CAUSAL else wl.Tq
    return gen_lact(wl.B, wl.H, Tq, Tkv, wl.d, wl.hid, seed=seed, dtype=wl.dtype)
