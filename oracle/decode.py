"""Single-token decode step of TTT-Linear in fp64 -- test infrastructure.

Like the rest of ``oracle/``, only tests, the smoke check and the benchmark's
CPU leg may use this module; the library never does.

Source: "Test-Time Training (TTT)" summary of *Learning to (Learn at Test
Time)*, "TTT definition" (the state carried from token to token, one gradient
step per token, the output read after the token's own step), examples 1 and 2
(inner-product and MSE losses with their gradients) and "Mini-batch gradient
descent" (inside a chunk every gradient is taken at the chunk-start state).

One call consumes one token per (batch, head):

    g     = k^T (k A - v)   (MSE)    or    -k^T v   (inner product)
    W'    = W - eta * g
    y     = q W'

where W is the carried (running) state and A the state the gradient is taken
at: A = W for the recurrent rule (chunk size 1); A = the state at the start of
the current chunk for chunked decoding, whose caller moves A to W' after the
chunk's last token.  Written per head with explicit fp64 vector operations;
no blocking or re-association beyond the formula.
"""
from __future__ import annotations

import numpy as np

LOSS_DOT = 0
LOSS_MSE = 1


def ttt_linear_decode(q, k, v, eta, w, w_anchor=None, *, loss: int, anchor_update: bool = False):
    """q, k, v [B,H,d]; eta [B,H]; w [B,H,d,d] (y = x W); w_anchor [B,H,d,d] or None.

    Returns (y [B,H,d], w_new [B,H,d,d], anchor_new or None).  anchor_new is
    w_new where anchor_update is set, else the anchor unchanged."""
    q, k, v, eta, w = (np.asarray(a, dtype=np.float64) for a in (q, k, v, eta, w))
    B, H, d = q.shape
    assert k.shape == (B, H, d) and v.shape == (B, H, d) and eta.shape == (B, H)
    assert w.shape == (B, H, d, d)
    anchor = None if w_anchor is None else np.array(w_anchor, dtype=np.float64)
    y = np.zeros((B, H, d))
    w_new = np.zeros_like(w)
    for b in range(B):
        for h in range(H):
            W = w[b, h]
            A = W if anchor is None else anchor[b, h]
            kv = k[b, h]
            if loss == LOSS_MSE:
                resid = kv @ A - v[b, h]          # d loss / d (k A)
            elif loss == LOSS_DOT:
                resid = -v[b, h]
            else:
                raise ValueError(loss)
            grad = np.outer(kv, resid)            # d loss / d W at A
            Wn = W - eta[b, h] * grad
            w_new[b, h] = Wn
            y[b, h] = q[b, h] @ Wn
            if anchor is not None and anchor_update:
                anchor[b, h] = Wn
    return y, w_new, anchor


def ttt_linear_decode_sequence(q, k, v, eta, w0, *, loss: int, chunk: int = 1):
    """Run T decode steps over q/k/v [B,H,T,d], eta [B,H,T] from w0, with the
    chunk-start anchor when chunk > 1 (moved at every chunk's last token).
    Returns (y [B,H,T,d], w_final)."""
    q, k, v, eta = (np.asarray(a, dtype=np.float64) for a in (q, k, v, eta))
    T = q.shape[2]
    w = np.array(w0, dtype=np.float64)
    anchor = None if chunk == 1 else w.copy()
    ys = []
    for t in range(T):
        last = (t + 1) % chunk == 0 or t == T - 1
        y, w, anchor = ttt_linear_decode(q[:, :, t], k[:, :, t], v[:, :, t], eta[:, :, t], w,
                                         anchor, loss=loss, anchor_update=last)
        ys.append(y)
    return np.stack(ys, axis=2), w
