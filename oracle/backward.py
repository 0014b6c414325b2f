"""Backward pass of the TTT-Linear forward in fp64 -- test infrastructure.

Like the rest of ``oracle/``, only tests, the smoke check and the benchmark's
CPU leg may use this module; the library never does.

The forward it differentiates is the token-by-token definition of
"Test-Time Training (TTT)" ("TTT definition", examples 1 and 2, "TTT-Linear",
"Mini-batch gradient descent"), with the readings of the forward oracle: per
chunk, every token's gradient is taken at the chunk-start state W_c,

    r_t = k_t W_c - v_t  (MSE)   or   -v_t  (inner product)
    W   <- W - eta_t k_t^T r_t          (running state, W = W_c at the chunk start)
    y_t = q_t W                          (after token t's own step)

and the final state is W after the last token.  Given upstream gradients
dy_t and dW_final, this is reverse-mode differentiation of exactly those
steps, token by token in reverse, each step's adjoint written out:

    y_t = q_t W_t            ->  dq_t = dy_t W_t^T,        dW_t += q_t^T dy_t
    W_t = W_{t-1} - eta_t k_t^T r_t
                             ->  dW_{t-1} += dW_t,
                                 d eta_t  = -k_t dW_t r_t^T,
                                 dk_t    += -eta_t dW_t r_t^T (as a row),
                                 dr_t     = -eta_t k_t dW_t
    r_t = k_t W_c - v_t      ->  dk_t += dr_t W_c^T,  dW_c += k_t^T dr_t,  dv_t = -dr_t
    r_t = -v_t               ->  dv_t = -dr_t

and at a chunk start the gradient reaching W_c (the running state before the
chunk's first token) adds the residual contributions dW_c.  The running states
W_t of a chunk are recomputed forward from W_c before its reverse sweep.  The
update-then-apply order (all key/value chunks update, then every query reads
the final state) is differentiated the same way, its apply first.
"""
from __future__ import annotations

import numpy as np

LOSS_DOT = 0
LOSS_MSE = 1


def _head_bwd_noncausal(q, k, v, eta, w0, dy, dwf, chunk, loss):
    """Update-then-apply order: the chunked updates run over all key/value tokens
    (no outputs), then y_j = q_j W_final for every query.  Adjoint of the apply:
    dq_j = dy_j W_final^T and dW_final += sum_j q_j^T dy_j; then the same reverse
    sweep over the key/value chunks with no output terms."""
    Tkv, d = k.shape
    W = w0.copy()
    for c0 in range(0, Tkv, chunk):
        Wc = W.copy()
        for t in range(c0, min(c0 + chunk, Tkv)):
            r = k[t] @ Wc - v[t] if loss == LOSS_MSE else -v[t]
            W = W - eta[t] * np.outer(k[t], r)
    dq = dy @ W.T
    G = dwf + q.T @ dy
    dk, dv, deta = np.zeros_like(k), np.zeros_like(v), np.zeros_like(eta)
    zero_q = np.zeros((Tkv, d))
    _, dk, dv, deta, G = _head_bwd(zero_q, k, v, eta, w0, zero_q, G, chunk, loss)
    return dq, dk, dv, deta, G


def _head_bwd(q, k, v, eta, w0, dy, dwf, chunk, loss):
    T, d = k.shape
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    deta = np.zeros_like(eta)
    # chunk-start states by the forward recursion
    starts = []
    W = w0.copy()
    for c0 in range(0, T, chunk):
        starts.append(W.copy())
        Wc = W.copy()
        for t in range(c0, min(c0 + chunk, T)):
            r = k[t] @ Wc - v[t] if loss == LOSS_MSE else -v[t]
            W = W - eta[t] * np.outer(k[t], r)
    G = dwf.copy()                      # gradient w.r.t. the running state after the last token
    for ci in range(len(starts) - 1, -1, -1):
        c0 = ci * chunk
        c1 = min(c0 + chunk, T)
        Wc = starts[ci]
        # running states W_t after each token of the chunk, and the residuals
        Ws, rs = [], []
        W = Wc.copy()
        for t in range(c0, c1):
            r = k[t] @ Wc - v[t] if loss == LOSS_MSE else -v[t]
            W = W - eta[t] * np.outer(k[t], r)
            Ws.append(W.copy())
            rs.append(r)
        dWc = np.zeros_like(Wc)         # residual contributions to the chunk-start state
        for i in range(c1 - c0 - 1, -1, -1):
            t = c0 + i
            Wt, r = Ws[i], rs[i]
            dq[t] = dy[t] @ Wt.T
            G = G + np.outer(q[t], dy[t])
            deta[t] = -(k[t] @ G @ r)
            dk[t] += -eta[t] * (G @ r)
            dr = -eta[t] * (k[t] @ G)
            if loss == LOSS_MSE:
                dk[t] += dr @ Wc.T
                dWc += np.outer(k[t], dr)
            dv[t] = -dr
            # the identity part of W_t = W_{t-1} - ... keeps G as it is
        G = G + dWc
    return dq, dk, dv, deta, G


def ttt_linear_bwd(q, k, v, eta, w0, dy, dwf=None, *, chunk: int, loss: int, order: int = 0):
    """q, dy [B,H,Tq,d]; k, v [B,H,Tkv,d]; eta [B,H,Tkv]; w0, dwf [B,H,d,d] (dwf None
    = zero).  order 0: causal (Tq == Tkv); 1: update over all keys, then apply to
    every query.  Returns (dq, dk, dv, deta, dw0)."""
    q, k, v, eta, w0, dy = (np.asarray(a, dtype=np.float64) for a in (q, k, v, eta, w0, dy))
    B, H, Tq, d = q.shape
    dwf = np.zeros((B, H, d, d)) if dwf is None else np.asarray(dwf, dtype=np.float64)
    outs = [np.zeros_like(q), np.zeros_like(k), np.zeros_like(v), np.zeros_like(eta),
            np.zeros_like(w0)]
    fn = _head_bwd if order == 0 else _head_bwd_noncausal
    for b in range(B):
        for h in range(H):
            r = fn(q[b, h], k[b, h], v[b, h], eta[b, h], w0[b, h], dy[b, h], dwf[b, h],
                   chunk, loss)
            for o, x in zip(outs, r):
                o[b, h] = x
    return tuple(outs)
