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


def _validate(device, *specs) -> None:
    """Full check of the tensors handed to the library, each spec being
    (tensor, name, shape, dtype): first every shape and dtype, then that every
    tensor is a contiguous GPU tensor on ``device``.  The C ABI only sees
    pointers, so a tensor that is too small or of the wrong type would be read
    or written out of bounds; everything is checked here before anything is
    enqueued."""
    for t, name, shape, dtype in specs:
        if t is None:
            raise ValueError(f"{name} is required")
        if tuple(t.shape) != tuple(shape):
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
        if t.dtype != dtype:
            raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    for t, name, _, dtype in specs:
        _check(t, name, dtype)
        if t.device != device:
            raise ValueError(f"{name} is on {t.device}, expected {device}")


def _workspace(ws: Optional[torch.Tensor], nbytes: int, device) -> torch.Tensor:
    """The caller's workspace if it is a large enough uint8 GPU buffer, else a new one."""
    if ws is None or ws.numel() < nbytes:
        return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)
    _check(ws, "workspace", torch.uint8)
    if ws.device != device:
        raise ValueError(f"workspace is on {ws.device}, expected {device}")
    return ws


_AUX = {}


def _aux_stream(aux, device) -> Optional[int]:
    """The second stream handed to the LaCT calls: "auto" = one torch stream per
    device (default priority) that this binding creates on first use; None = no
    second stream; else a torch.cuda.Stream of the caller's."""
    if aux is None:
        return None
    if isinstance(aux, str):
        if aux != "auto":
            raise ValueError("aux_stream must be 'auto', None or a torch.cuda.Stream")
        idx = device.index if device.index is not None else torch.cuda.current_device()
        if idx not in _AUX:
            _AUX[idx] = torch.cuda.Stream(device=idx)
        aux = _AUX[idx]
    return aux.cuda_stream


def _stream(stream) -> int:
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def ttt_linear_workspace_bytes(B, H, Tq, Tkv, d, chunk, loss, order, dtype, seg_tokens=0) -> int:
    return int(load().ttt_linear_workspace_bytes_seg(B, H, Tq, Tkv, d, chunk, _LOSS[loss],
                                                     _ORDER[order], _DT[dtype], int(seg_tokens)))


def _dims(t: torch.Tensor, n: int, name: str):
    if t.dim() != n:
        raise ValueError(f"{name} must have {n} dimensions, got {t.dim()}")
    return tuple(t.shape)


def ttt_linear_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, eta: torch.Tensor,
                   w_init: torch.Tensor, *, chunk: int, loss="mse", order="causal",
                   out: Optional[torch.Tensor] = None, w_final: Optional[torch.Tensor] = None,
                   workspace: Optional[torch.Tensor] = None, seg_tokens: int = 0,
                   stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """TTT-Linear forward.  Returns (out [B,H,Tq,d], w_final [B,H,d,d]).
    ``seg_tokens`` > 0 sets the segment length of the state scan (ttt_linear_fwd_seg);
    0 leaves it to the library."""
    lib = load()
    B, H, Tq, d = _dims(q, 4, "q")
    Tkv = _dims(k, 4, "k")[2]
    dt, dev = q.dtype, q.device
    if out is None:
        out = torch.empty_like(q)
    if w_final is None:
        w_final = torch.empty_like(w_init)
    _validate(dev, (q, "q", (B, H, Tq, d), dt), (k, "k", (B, H, Tkv, d), dt),
              (v, "v", (B, H, Tkv, d), dt), (eta, "eta", (B, H, Tkv), torch.float32),
              (w_init, "w_init", (B, H, d, d), torch.float32), (out, "out", (B, H, Tq, d), dt),
              (w_final, "w_final", (B, H, d, d), torch.float32))
    ls, od = _LOSS[loss], _ORDER[order]
    nbytes = lib.ttt_linear_workspace_bytes_seg(B, H, Tq, Tkv, d, chunk, ls, od, _DT[dt],
                                                int(seg_tokens))
    workspace = _workspace(workspace, nbytes, dev)
    rc = lib.ttt_linear_fwd_seg(_ptr(q), _ptr(k), _ptr(v), _DT[dt], _ptr(eta), _ptr(w_init),
                                _ptr(out), _ptr(w_final), B, H, Tq, Tkv, d, chunk, ls, od,
                                int(seg_tokens), _ptr(workspace), workspace.numel(),
                                _stream(stream))
    if rc != TTT_OK:
        raise TTTError(rc, "ttt_linear_fwd")
    return out, w_final


def lact_swiglu_workspace_bytes(B, H, Tq, Tkv, d, hidden, chunk, loss, order, dtype) -> int:
    return int(load().lact_swiglu_workspace_bytes(B, H, Tq, Tkv, d, hidden, chunk, _LOSS[loss],
                                                  _ORDER[order], _DT[dtype]))


def _lact_dims(q, k, v, eta, w1, w2, w3):
    """Shapes of a LaCT call (checked against every tensor by _lact_specs)."""
    B, H, Tq, d = _dims(q, 4, "q")
    Tkv = _dims(k, 4, "k")[2]
    hid = _dims(w1, 4, "w1")[2]
    return B, H, Tq, d, Tkv, hid, q.dtype, q.device


def _lact_outs(q, w1, w2, w3, out, w1_final, w2_final, w3_final):
    """Output tensors of a LaCT call (new ones where the caller gave none)."""
    out = torch.empty_like(q) if out is None else out
    w1_final = torch.empty_like(w1) if w1_final is None else w1_final
    w2_final = torch.empty_like(w2) if w2_final is None else w2_final
    w3_final = torch.empty_like(w3) if w3_final is None else w3_final
    return out, w1_final, w2_final, w3_final


def _lact_specs(B, H, Tq, d, Tkv, hid, dt, q, k, v, eta, w1, w2, w3, out, w1f, w2f, w3f):
    """(tensor, name, shape, dtype) of every tensor of a LaCT call, for _validate."""
    f = torch.float32
    return ((q, "q", (B, H, Tq, d), dt), (k, "k", (B, H, Tkv, d), dt),
            (v, "v", (B, H, Tkv, d), dt), (eta, "eta", (B, H, Tkv), f),
            (w1, "w1", (B, H, hid, d), f), (w2, "w2", (B, H, d, hid), f),
            (w3, "w3", (B, H, hid, d), f), (out, "out", (B, H, Tq, d), dt),
            (w1f, "w1_final", (B, H, hid, d), f), (w2f, "w2_final", (B, H, d, hid), f),
            (w3f, "w3_final", (B, H, hid, d), f))


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
                         w2_final=None, w3_final=None, workspace=None, stream=None,
                         aux_stream="auto"):
    """LaCT SwiGLU forward with an update rule ("gd", "momentum", "muon").
    ``momentum`` = (m1, m2, m3) fp32 buffers shaped like the weights, updated in
    place (needed by "momentum", and by "muon" when beta != 0).  ``aux_stream``:
    the second stream the causal applies may use ("auto", None or a stream).
    Returns (out, w1_final, w2_final, w3_final)."""
    lib = load()
    B, H, Tq, d, Tkv, hid, dt, dev = _lact_dims(q, k, v, eta, w1, w2, w3)
    ms = (None, None, None) if momentum is None else tuple(momentum)
    if len(ms) != 3:
        raise ValueError("momentum must be (m1, m2, m3)")
    out, w1_final, w2_final, w3_final = _lact_outs(q, w1, w2, w3, out, w1_final, w2_final,
                                                   w3_final)
    specs = _lact_specs(B, H, Tq, d, Tkv, hid, dt, q, k, v, eta, w1, w2, w3, out, w1_final,
                        w2_final, w3_final)
    specs += tuple((t, n, tuple(w.shape), torch.float32)
                   for t, w, n in zip(ms, (w1, w2, w3), ("m1", "m2", "m3")) if t is not None)
    _validate(dev, *specs)
    ls, od, ru = _LOSS[loss], _ORDER[order], _RULE[rule]
    nbytes = lib.lact_swiglu_rule_workspace_bytes(B, H, Tq, Tkv, d, hid, chunk, ls, od, _DT[dt], ru)
    workspace = _workspace(workspace, nbytes, dev)
    rc = lib.lact_swiglu_fwd_rule(_ptr(q), _ptr(k), _ptr(v), _DT[dt], _ptr(eta), _ptr(w1),
                                  _ptr(w2), _ptr(w3), _ptr(out), _ptr(w1_final), _ptr(w2_final),
                                  _ptr(w3_final), B, H, Tq, Tkv, d, hid, chunk, ls, od,
                                  int(bool(rownorm)), ru, float(beta), int(ns_steps),
                                  float(muon_lr), _ptr(ms[0]), _ptr(ms[1]), _ptr(ms[2]),
                                  _ptr(workspace), workspace.numel(), _stream(stream),
                                  _aux_stream(aux_stream, dev))
    if rc != TTT_OK:
        raise TTTError(rc, "lact_swiglu_fwd_rule")
    return out, w1_final, w2_final, w3_final


def lact_swiglu_fwd(q, k, v, eta, w1, w2, w3, *, chunk: int, loss="dot", order="causal",
                    rownorm: bool = True, out=None, w1_final=None, w2_final=None, w3_final=None,
                    workspace=None, stream=None, aux_stream="auto"):
    """LaCT SwiGLU forward.  ``aux_stream``: the second stream the causal applies
    may use ("auto": one per device, made by this binding; None: none; or a
    torch.cuda.Stream).  Returns (out, w1_final, w2_final, w3_final)."""
    lib = load()
    B, H, Tq, d, Tkv, hid, dt, dev = _lact_dims(q, k, v, eta, w1, w2, w3)
    out, w1_final, w2_final, w3_final = _lact_outs(q, w1, w2, w3, out, w1_final, w2_final,
                                                   w3_final)
    _validate(dev, *_lact_specs(B, H, Tq, d, Tkv, hid, dt, q, k, v, eta, w1, w2, w3, out,
                                w1_final, w2_final, w3_final))
    ls, od = _LOSS[loss], _ORDER[order]
    nbytes = lib.lact_swiglu_workspace_bytes(B, H, Tq, Tkv, d, hid, chunk, ls, od, _DT[dt])
    workspace = _workspace(workspace, nbytes, dev)
    rc = lib.lact_swiglu_fwd(_ptr(q), _ptr(k), _ptr(v), _DT[dt], _ptr(eta), _ptr(w1), _ptr(w2),
                             _ptr(w3), _ptr(out), _ptr(w1_final), _ptr(w2_final), _ptr(w3_final),
                             B, H, Tq, Tkv, d, hid, chunk, ls, od, int(bool(rownorm)),
                             _ptr(workspace), workspace.numel(), _stream(stream),
                             _aux_stream(aux_stream, dev))
    if rc != TTT_OK:
        raise TTTError(rc, "lact_swiglu_fwd")
    return out, w1_final, w2_final, w3_final


def ttt_linear_decode(q, k, v, eta, w, *, loss="mse", w_anchor=None, anchor_update=False,
                      out=None, stream=None):
    """One decode step: q, k, v [B,H,d], eta [B,H]; w [B,H,d,d] fp32 is updated in
    place; w_anchor (optional, [B,H,d,d] fp32) is the chunk-start state, moved to
    the new state when anchor_update is set.  Returns out [B,H,d]."""
    lib = load()
    B, H, d = _dims(q, 3, "q")
    dt, dev = q.dtype, q.device
    out = torch.empty_like(q) if out is None else out
    specs = [(q, "q", (B, H, d), dt), (k, "k", (B, H, d), dt), (v, "v", (B, H, d), dt),
             (eta, "eta", (B, H), torch.float32), (w, "w", (B, H, d, d), torch.float32),
             (out, "out", (B, H, d), dt)]
    if w_anchor is not None:
        specs.append((w_anchor, "w_anchor", (B, H, d, d), torch.float32))
    _validate(dev, *specs)
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
    B, H, d = _dims(q, 3, "q")
    hid = _dims(w1, 4, "w1")[2]
    dt, dev = q.dtype, q.device
    out = torch.empty_like(q) if out is None else out
    _validate(dev, (q, "q", (B, H, d), dt), (w1, "w1", (B, H, hid, d), torch.float32),
              (w2, "w2", (B, H, d, hid), torch.float32), (w3, "w3", (B, H, hid, d), torch.float32),
              (out, "out", (B, H, d), dt))
    nbytes = lib.lact_swiglu_decode_workspace_bytes(B, H, d, hid, _DT[dt])
    workspace = _workspace(workspace, nbytes, dev)
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
    B, H, T, d = _dims(q, 4, "q")
    dt, dev = q.dtype, q.device
    if out is None:
        if accumulate:
            raise ValueError("accumulate needs out")
        out = torch.empty_like(q)
    _validate(dev, *((t, n, (B, H, T, d), dt) for t, n in ((q, "q"), (k, "k"), (v, "v"), (out, "out"))))
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
    B, H, Tq, d = _dims(q, 4, "q")
    Tkv = _dims(k, 4, "k")[2]
    dt, dev = q.dtype, q.device
    specs = [(t, n, (B, H, T, d), dt)
             for t, n, T in ((q, "q", Tq), (k, "k", Tkv), (v, "v", Tkv), (d_out, "d_out", Tq))]
    specs += [(eta, "eta", (B, H, Tkv), torch.float32),
              (w_init, "w_init", (B, H, d, d), torch.float32)]
    if d_w_final is not None:
        specs.append((d_w_final, "d_w_final", (B, H, d, d), torch.float32))
    _validate(dev, *specs)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    deta, dw0 = torch.empty_like(eta), torch.empty_like(w_init)
    ls, od = _LOSS[loss], _ORDER[order]
    nbytes = lib.ttt_linear_bwd_workspace_bytes(B, H, Tq, Tkv, d, chunk, ls, od, _DT[dt])
    workspace = _workspace(workspace, nbytes, dev)
    rc = lib.ttt_linear_bwd(_ptr(q), _ptr(k), _ptr(v), _DT[dt], _ptr(eta), _ptr(w_init),
                            _ptr(d_out), _ptr(d_w_final), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(deta),
                            _ptr(dw0), B, H, Tq, Tkv, d, chunk, ls, od, _ptr(workspace),
                            workspace.numel(), _stream(stream))
    if rc != TTT_OK:
        raise TTTError(rc, "ttt_linear_bwd")
    return dq, dk, dv, deta, dw0


def lact_swiglu_bwd(q, k, v, eta, w1, w2, w3, d_out, d_w_final=None, *, chunk: int, loss="dot",
                    order="causal", rownorm: bool = True, workspace=None, stream=None):
    """Backward of lact_swiglu_fwd (inner-product loss, gradient descent): returns
    (d_q, d_k, d_v, d_eta, d_w1, d_w2, d_w3) for upstream gradients d_out
    [B,H,Tq,d] (q's dtype) and d_w_final = (d_w1, d_w2, d_w3) fp32 shaped like the
    weights (None = zero)."""
    lib = load()
    B, H, Tq, d, Tkv, hid, dt, dev = _lact_dims(q, k, v, eta, w1, w2, w3)
    specs = list(_lact_specs(B, H, Tq, d, Tkv, hid, dt, q, k, v, eta, w1, w2, w3, q, w1, w2,
                             w3))[:7]
    specs.append((d_out, "d_out", (B, H, Tq, d), dt))
    if d_w_final is not None:
        if len(d_w_final) != 3:
            raise ValueError("d_w_final must be (d_w1, d_w2, d_w3)")
        specs += [(t, n, tuple(w.shape), torch.float32)
                  for t, w, n in zip(d_w_final, (w1, w2, w3), ("d_w1_final", "d_w2_final",
                                                               "d_w3_final"))]
    _validate(dev, *specs)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    deta = torch.empty_like(eta)
    dw1, dw2, dw3 = torch.empty_like(w1), torch.empty_like(w2), torch.empty_like(w3)
    ls, od = _LOSS[loss], _ORDER[order]
    nbytes = lib.lact_swiglu_bwd_workspace_bytes(B, H, Tq, Tkv, d, hid, chunk, ls, od, _DT[dt])
    workspace = _workspace(workspace, nbytes, dev)
    dwf = (None, None, None) if d_w_final is None else tuple(d_w_final)
    rc = lib.lact_swiglu_bwd(_ptr(q), _ptr(k), _ptr(v), _DT[dt], _ptr(eta), _ptr(w1), _ptr(w2),
                             _ptr(w3), _ptr(d_out), _ptr(dwf[0]), _ptr(dwf[1]), _ptr(dwf[2]),
                             _ptr(dq), _ptr(dk), _ptr(dv), _ptr(deta), _ptr(dw1), _ptr(dw2),
                             _ptr(dw3), B, H, Tq, Tkv, d, hid, chunk, ls, od, int(bool(rownorm)),
                             _ptr(workspace), workspace.numel(), _stream(stream))
    if rc != TTT_OK:
        raise TTTError(rc, "lact_swiglu_bwd")
    return dq, dk, dv, deta, dw1, dw2, dw3
