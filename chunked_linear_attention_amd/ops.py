"""Python entry points with the C ABI's names: marshalling only.

Tensors follow include/ttt.h: q [B,H,Tq,d], k/v [B,H,Tkv,d] (bf16 or fp32,
contiguous, on the GPU), eta [B,H,Tkv] fp32, states fp32.
"""
from __future__ import annotations

from typing import Optional, Tuple

import torch

from ._lib import TTT_OK, TTTError, load

LOSS_DOT, LOSS_MSE = 0, 1
CAUSAL, NONCAUSAL = 0, 1
_DT = {torch.float32: 0, torch.bfloat16: 1}
_LOSS = {"dot": LOSS_DOT, "inner": LOSS_DOT, "mse": LOSS_MSE, LOSS_DOT: LOSS_DOT, LOSS_MSE: LOSS_MSE}
_ORDER = {"causal": CAUSAL, "noncausal": NONCAUSAL, "non-causal": NONCAUSAL, CAUSAL: CAUSAL,
          NONCAUSAL: NONCAUSAL}


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _check(t: torch.Tensor, name: str, dtype=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")


def _stream(stream) -> int:
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def ttt_linear_workspace_bytes(B, H, Tq, Tkv, d, chunk, loss, order, dtype) -> int:
    return int(load().ttt_linear_workspace_bytes(B, H, Tq, Tkv, d, chunk, _LOSS[loss],
                                                 _ORDER[order], _DT[dtype]))


def ttt_linear_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, eta: torch.Tensor,
                   w_init: torch.Tensor, *, chunk: int, loss="mse", order="causal",
                   out: Optional[torch.Tensor] = None, w_final: Optional[torch.Tensor] = None,
                   workspace: Optional[torch.Tensor] = None,
                   stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """TTT-Linear forward.  Returns (out [B,H,Tq,d], w_final [B,H,d,d])."""
    lib = load()
    B, H, Tq, d = q.shape
    Tkv = k.shape[2]
    dt = q.dtype
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _check(t, n, dt)
    _check(eta, "eta", torch.float32)
    _check(w_init, "w_init", torch.float32)
    if out is None:
        out = torch.empty_like(q)
    if w_final is None:
        w_final = torch.empty_like(w_init)
    ls, od = _LOSS[loss], _ORDER[order]
    nbytes = lib.ttt_linear_workspace_bytes(B, H, Tq, Tkv, d, chunk, ls, od, _DT[dt])
    if workspace is None or workspace.numel() < nbytes:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    rc = lib.ttt_linear_fwd(_ptr(q), _ptr(k), _ptr(v), _DT[dt], _ptr(eta), _ptr(w_init), _ptr(out),
                            _ptr(w_final), B, H, Tq, Tkv, d, chunk, ls, od, _ptr(workspace),
                            workspace.numel(), _stream(stream))
    if rc != TTT_OK:
        raise TTTError(rc, "ttt_linear_fwd")
    return out, w_final


def lact_swiglu_workspace_bytes(B, H, Tq, Tkv, d, hidden, chunk, loss, order, dtype) -> int:
    return int(load().lact_swiglu_workspace_bytes(B, H, Tq, Tkv, d, hidden, chunk, _LOSS[loss],
                                                  _ORDER[order], _DT[dtype]))


RULE_GD, RULE_MOMENTUM, RULE_MUON = 0, 1, 2
_RULE = {"gd": RULE_GD, "momentum": RULE_MOMENTUM, "muon": RULE_MUON, RULE_GD: RULE_GD,
         RULE_MOMENTUM: RULE_MOMENTUM, RULE_MUON: RULE_MUON}


def lact_swiglu_rule_workspace_bytes(B, H, Tq, Tkv, d, hidden, chunk, loss, order, dtype,
                                     rule) -> int:
    return int(load().lact_swiglu_rule_workspace_bytes(B, H, Tq, Tkv, d, hidden, chunk,
                                                       _LOSS[loss], _ORDER[order], _DT[dtype],
                                                       _RULE[rule]))


def lact_swiglu_fwd_rule(q, k, v, eta, w1, w2, w3, *, chunk: int, rule="gd", beta: float = 0.0,
                         ns_steps: int = 5, muon_lr: float = 0.0, momentum=None, loss="dot",
                         order="causal", rownorm: bool = True, out=None, w1_final=None,
                         w2_final=None, w3_final=None, workspace=None, stream=None):
    """LaCT SwiGLU forward with an update rule ("gd", "momentum", "muon").
    ``momentum`` = (m1, m2, m3) fp32 buffers shaped like the weights, updated in
    place (needed by "momentum", and by "muon" when beta != 0).
    Returns (out, w1_final, w2_final, w3_final)."""
    lib = load()
    B, H, Tq, d = q.shape
    Tkv = k.shape[2]
    hid = w1.shape[2]
    dt = q.dtype
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _check(t, n, dt)
    _check(eta, "eta", torch.float32)
    for t, n in ((w1, "w1"), (w2, "w2"), (w3, "w3")):
        _check(t, n, torch.float32)
    ms = (None, None, None) if momentum is None else tuple(momentum)
    for t, w, n in zip(ms, (w1, w2, w3), ("m1", "m2", "m3")):
        if t is not None:
            _check(t, n, torch.float32)
            if t.shape != w.shape:
                raise ValueError(f"{n} must be shaped like its weight")
    out = torch.empty_like(q) if out is None else out
    w1_final = torch.empty_like(w1) if w1_final is None else w1_final
    w2_final = torch.empty_like(w2) if w2_final is None else w2_final
    w3_final = torch.empty_like(w3) if w3_final is None else w3_final
    ls, od, ru = _LOSS[loss], _ORDER[order], _RULE[rule]
    nbytes = lib.lact_swiglu_rule_workspace_bytes(B, H, Tq, Tkv, d, hid, chunk, ls, od, _DT[dt], ru)
    if workspace is None or workspace.numel() < nbytes:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    rc = lib.lact_swiglu_fwd_rule(_ptr(q), _ptr(k), _ptr(v), _DT[dt], _ptr(eta), _ptr(w1),
                                  _ptr(w2), _ptr(w3), _ptr(out), _ptr(w1_final), _ptr(w2_final),
                                  _ptr(w3_final), B, H, Tq, Tkv, d, hid, chunk, ls, od,
                                  int(bool(rownorm)), ru, float(beta), int(ns_steps),
                                  float(muon_lr), _ptr(ms[0]), _ptr(ms[1]), _ptr(ms[2]),
                                  _ptr(workspace), workspace.numel(), _stream(stream))
    if rc != TTT_OK:
        raise TTTError(rc, "lact_swiglu_fwd_rule")
    return out, w1_final, w2_final, w3_final


def lact_swiglu_fwd(q, k, v, eta, w1, w2, w3, *, chunk: int, loss="dot", order="causal",
                    rownorm: bool = True, out=None, w1_final=None, w2_final=None, w3_final=None,
                    workspace=None, stream=None):
    """LaCT SwiGLU forward.  Returns (out, w1_final, w2_final, w3_final)."""
    lib = load()
    B, H, Tq, d = q.shape
    Tkv = k.shape[2]
    hid = w1.shape[2]
    dt = q.dtype
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _check(t, n, dt)
    _check(eta, "eta", torch.float32)
    for t, n in ((w1, "w1"), (w2, "w2"), (w3, "w3")):
        _check(t, n, torch.float32)
    out = torch.empty_like(q) if out is None else out
    w1_final = torch.empty_like(w1) if w1_final is None else w1_final
    w2_final = torch.empty_like(w2) if w2_final is None else w2_final
    w3_final = torch.empty_like(w3) if w3_final is None else w3_final
    ls, od = _LOSS[loss], _ORDER[order]
    nbytes = lib.lact_swiglu_workspace_bytes(B, H, Tq, Tkv, d, hid, chunk, ls, od, _DT[dt])
    if workspace is None or workspace.numel() < nbytes:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    rc = lib.lact_swiglu_fwd(_ptr(q), _ptr(k), _ptr(v), _DT[dt], _ptr(eta), _ptr(w1), _ptr(w2),
                             _ptr(w3), _ptr(out), _ptr(w1_final), _ptr(w2_final), _ptr(w3_final),
                             B, H, Tq, Tkv, d, hid, chunk, ls, od, int(bool(rownorm)),
                             _ptr(workspace), workspace.numel(), _stream(stream))
    if rc != TTT_OK:
        raise TTTError(rc, "lact_swiglu_fwd")
    return out, w1_final, w2_final, w3_final


def ttt_linear_decode(q, k, v, eta, w, *, loss="mse", w_anchor=None, anchor_update=False,
                      out=None, stream=None):
    """One decode step: q, k, v [B,H,d], eta [B,H]; w [B,H,d,d] fp32 is updated in
    place; w_anchor (optional, [B,H,d,d] fp32) is the chunk-start state, moved to
    the new state when anchor_update is set.  Returns out [B,H,d]."""
    lib = load()
    B, H, d = q.shape
    dt = q.dtype
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _check(t, n, dt)
    _check(eta, "eta", torch.float32)
    _check(w, "w", torch.float32)
    if w_anchor is not None:
        _check(w_anchor, "w_anchor", torch.float32)
    if tuple(k.shape) != (B, H, d) or tuple(v.shape) != (B, H, d) or tuple(eta.shape) != (B, H) \
            or tuple(w.shape) != (B, H, d, d) or (w_anchor is not None and w_anchor.shape != w.shape):
        raise ValueError("ttt_linear_decode: inconsistent shapes")
    out = torch.empty_like(q) if out is None else out
    rc = lib.ttt_linear_decode(_ptr(q), _ptr(k), _ptr(v), _DT[dt], _ptr(eta), _ptr(w),
                               _ptr(w_anchor), int(bool(anchor_update)), _ptr(out), B, H, d,
                               _LOSS[loss], _stream(stream))
    if rc != TTT_OK:
        raise TTTError(rc, "ttt_linear_decode")
    return out


def lact_swiglu_decode_workspace_bytes(B, H, d, hidden, dtype) -> int:
    return int(load().lact_swiglu_decode_workspace_bytes(B, H, d, hidden, _DT[dtype]))


def lact_swiglu_decode(q, w1, w2, w3, *, out=None, workspace=None, stream=None):
    """LaCT decode apply: q [B,H,d] -> W2 (silu(W1 q) * (W3 q)) [B,H,d] with the
    weights as they stand (w1, w3 [B,H,hid,d], w2 [B,H,d,hid] fp32)."""
    lib = load()
    B, H, d = q.shape
    hid = w1.shape[2]
    dt = q.dtype
    _check(q, "q", dt)
    for t, n in ((w1, "w1"), (w2, "w2"), (w3, "w3")):
        _check(t, n, torch.float32)
    if tuple(w1.shape) != (B, H, hid, d) or w3.shape != w1.shape or tuple(w2.shape) != (B, H, d, hid):
        raise ValueError("lact_swiglu_decode: inconsistent shapes")
    out = torch.empty_like(q) if out is None else out
    nbytes = lib.lact_swiglu_decode_workspace_bytes(B, H, d, hid, _DT[dt])
    if workspace is None or workspace.numel() < nbytes:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    rc = lib.lact_swiglu_decode(_ptr(q), _DT[dt], _ptr(w1), _ptr(w2), _ptr(w3), _ptr(out), B, H, d,
                                hid, _ptr(workspace), workspace.numel(), _stream(stream))
    if rc != TTT_OK:
        raise TTTError(rc, "lact_swiglu_decode")
    return out


def window_attention_fwd(q, k, v, *, window: int, scale=None, out=None, accumulate=False,
                         stream=None):
    """Causal sliding-window softmax attention over q, k, v [B,H,T,d] (bf16): query t
    attends to keys t - window < s <= t with scores scale * q.k (scale 1/sqrt(d) by
    default).  With accumulate, adds into ``out`` (e.g. the LaCT output).  Returns out."""
    lib = load()
    B, H, T, d = q.shape
    dt = q.dtype
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _check(t, n, dt)
        if tuple(t.shape) != (B, H, T, d):
            raise ValueError(f"{n} must be shaped like q")
    if out is None:
        if accumulate:
            raise ValueError("accumulate needs out")
        out = torch.empty_like(q)
    _check(out, "out", dt)
    sc = float(d) ** -0.5 if scale is None else float(scale)
    rc = lib.window_attention_fwd(_ptr(q), _ptr(k), _ptr(v), _DT[dt], _ptr(out), B, H, T, d,
                                  int(window), sc, int(bool(accumulate)), _stream(stream))
    if rc != TTT_OK:
        raise TTTError(rc, "window_attention_fwd")
    return out


def ttt_linear_bwd(q, k, v, eta, w_init, d_out, d_w_final=None, *, chunk: int, loss="mse",
                   order="causal", workspace=None, stream=None):
    """Backward of ttt_linear_fwd: returns (d_q, d_k, d_v, d_eta, d_w_init) for
    upstream gradients d_out [B,H,Tq,d] (q's dtype) and d_w_final [B,H,d,d] fp32
    (None = zero)."""
    lib = load()
    B, H, Tq, d = q.shape
    Tkv = k.shape[2]
    dt = q.dtype
    for t, n, T in ((q, "q", Tq), (k, "k", Tkv), (v, "v", Tkv), (d_out, "d_out", Tq)):
        _check(t, n, dt)
        if tuple(t.shape) != (B, H, T, d):
            raise ValueError(f"{n} has the wrong shape")
    _check(eta, "eta", torch.float32)
    _check(w_init, "w_init", torch.float32)
    if d_w_final is not None:
        _check(d_w_final, "d_w_final", torch.float32)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    deta, dw0 = torch.empty_like(eta), torch.empty_like(w_init)
    ls, od = _LOSS[loss], _ORDER[order]
    nbytes = lib.ttt_linear_bwd_workspace_bytes(B, H, Tq, Tkv, d, chunk, ls, od, _DT[dt])
    if workspace is None or workspace.numel() < nbytes:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    rc = lib.ttt_linear_bwd(_ptr(q), _ptr(k), _ptr(v), _DT[dt], _ptr(eta), _ptr(w_init),
                            _ptr(d_out), _ptr(d_w_final), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(deta),
                            _ptr(dw0), B, H, Tq, Tkv, d, chunk, ls, od, _ptr(workspace),
                            workspace.numel(), _stream(stream))
    if rc != TTT_OK:
        raise TTTError(rc, "ttt_linear_bwd")
    return dq, dk, dv, deta, dw0
