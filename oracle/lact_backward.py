"""LaCT SwiGLU backward: reverse-mode differentiation of the chunked forward.

Test infrastructure, like the rest of ``oracle/``: only tests, the smoke
check and the benchmark's CPU baseline call it.

What is differentiated ("LaCT: Test-Time Training Done Right", sections 3.2,
3.3 and 4; the same definitions as ``oracle.dense.lact_head``): per (batch,
head), fast weight f(x) = W2 (silu(W1 x) * (W3 x)); per chunk c of key tokens
the gradient D_c of sum_t eta_t L_t with the inner-product loss
L_t = -f(k_t) . v_t, taken at the chunk-start weights W_c, a gradient step
U = W_c - D_c and (optionally) every row back to its pre-update L2 norm,
W_{c+1}[r] = U[r] |W_c[r]| / |U[r]|.  Causal order: the queries of chunk c read
W_c; non-causal: every query reads the final weights.  The pages train the
layer end to end (their throughput figures are training throughputs, section
6, Table 3) but give no backward algorithm; this is reverse mode of exactly
the forward's steps, with upstream gradients dO (of the outputs) and dW (of
the final weights, or zero), for the scalar L = sum dO * O + sum_i dW_i * W_i,final.

Scope: the inner-product loss (the loss of the LaCT workloads) and gradient
descent.

Notation, rows are tokens: X [n, d]; H1 = X W1^T, H3 = X W3^T, S = sigmoid(H1),
A = silu(H1) = H1 S, A' = silu'(H1) = S (1 + H1 (1 - S)),
A'' = silu''(H1) = S (1 - S) (2 + H1 (1 - 2 S)), G = A * H3.

The chunk gradient (forward):   dY = -eta V,  dG = dY W2,  dH3 = dG * A,
dH1 = dG * H3 * A',  D1 = dH1^T K,  D3 = dH3^T K,  D2 = dY^T G.

Its reverse (given adjoints Gam1, Gam2, Gam3 of D1, D2, D3):
  P1 = K Gam1^T,  P3 = K Gam3^T,  P2 = dY Gam2          (adjoints of dH1, dH3, G)
  bar_dG = P1 * H3 * A' + P3 * A
  bar_H3 = P1 * dG * A' + P2 * A
  bar_H1 = P1 * dG * H3 * A'' + (P3 * dG + P2 * H3) * A'
  bar_W1 = bar_H1^T K,  bar_W3 = bar_H3^T K,  bar_W2 = dY^T bar_dG
  bar_K  = dH1 Gam1 + dH3 Gam3 + bar_H1 W1 + bar_H3 W3
  bar_dY = G Gam2^T + bar_dG W2^T,  bar_V = -eta * bar_dY,
  bar_eta = -rowsum(bar_dY * V)

The apply's reverse (rows X, upstream dO):
  bar_G = dO W2,  bar_W2 = dO^T G,  bar_H3 = bar_G * A,  bar_H1 = bar_G * H3 * A',
  bar_W1 = bar_H1^T X,  bar_W3 = bar_H3^T X,  bar_X = bar_H1 W1 + bar_H3 W3

The step's reverse, per row r, with n = |W_c[r]|, m = |U[r]|, s = n / m and
Lam the adjoint of W_{c+1}[r]:
  bar_U = s Lam - (U . Lam) n U / m^3,   bar_W_c += bar_U + (U . Lam) / m * W_c[r] / n
(without the row rescale: bar_U = Lam, bar_W_c += Lam), and Gam = -bar_U.
"""
from __future__ import annotations

import numpy as np


def _sig(z):
    return 1.0 / (1.0 + np.exp(-z))


def _act(h1):
    s = _sig(h1)
    a = h1 * s
    a1 = s * (1.0 + h1 * (1.0 - s))
    a2 = s * (1.0 - s) * (2.0 + h1 * (1.0 - 2.0 * s))
    return a, a1, a2


def _apply_fwd(x, w1, w2, w3):
    h1 = x @ w1.T
    h3 = x @ w3.T
    a, _, _ = _act(h1)
    return (a * h3) @ w2.T


def _apply_bwd(x, dout, w1, w2, w3):
    """Adjoints (bar_x, bar_w1, bar_w2, bar_w3) of sum dout * f(x)."""
    h1 = x @ w1.T
    h3 = x @ w3.T
    a, a1, _ = _act(h1)
    g = a * h3
    bg = dout @ w2
    bw2 = dout.T @ g
    bh3 = bg * a
    bh1 = bg * h3 * a1
    return bh1 @ w1 + bh3 @ w3, bh1.T @ x, bw2, bh3.T @ x


def _chunk_grad(k, v, eta, w1, w2, w3):
    """The chunk gradient D1, D2, D3 (inner-product loss) and what its reverse needs."""
    h1 = k @ w1.T
    h3 = k @ w3.T
    a, a1, a2 = _act(h1)
    g = a * h3
    dy = -eta[:, None] * v
    dg = dy @ w2
    dh3 = dg * a
    dh1 = dg * h3 * a1
    return (dh1.T @ k, dy.T @ g, dh3.T @ k), (h1, h3, a, a1, a2, g, dy, dg, dh1, dh3)


def _chunk_grad_bwd(k, v, eta, w1, w2, w3, gam, saved):
    """Adjoints (bar_w1, bar_w2, bar_w3, bar_k, bar_v, bar_eta) of
    sum_i gam_i * D_i(k, v, eta, w)."""
    gam1, gam2, gam3 = gam
    h1, h3, a, a1, a2, g, dy, dg, dh1, dh3 = saved
    p1 = k @ gam1.T
    p3 = k @ gam3.T
    p2 = dy @ gam2
    bdg = p1 * h3 * a1 + p3 * a
    bh3 = p1 * dg * a1 + p2 * a
    bh1 = p1 * dg * h3 * a2 + (p3 * dg + p2 * h3) * a1
    bw1 = bh1.T @ k
    bw3 = bh3.T @ k
    bw2 = dy.T @ bdg
    bk = dh1 @ gam1 + dh3 @ gam3 + bh1 @ w1 + bh3 @ w3
    bdy = g @ gam2.T + bdg @ w2.T
    bv = -eta[:, None] * bdy
    beta_ = -np.sum(bdy * v, axis=1)
    return bw1, bw2, bw3, bk, bv, beta_


def _step(w, d, rownorm):
    u = w - d
    if not rownorm:
        return u
    n = np.sqrt(np.sum(w * w, axis=1))
    m = np.sqrt(np.sum(u * u, axis=1))
    f = np.where(m == 0.0, 1.0, n / np.where(m == 0.0, 1.0, m))
    return u * f[:, None]


def _step_bwd(w, d, lam, rownorm):
    """(bar_w through the step's direct path, bar_U) for the adjoint lam of the
    stepped weight."""
    if not rownorm:
        return lam.copy(), lam.copy()
    u = w - d
    n = np.sqrt(np.sum(w * w, axis=1))
    m = np.sqrt(np.sum(u * u, axis=1))
    ul = np.sum(u * lam, axis=1)
    live = m > 0.0
    ms = np.where(live, m, 1.0)
    ns = np.where(n > 0.0, n, 1.0)
    s = np.where(live, n / ms, 1.0)
    bu = s[:, None] * lam - np.where(live, ul * n / ms ** 3, 0.0)[:, None] * u
    bw_norm = np.where(live & (n > 0.0), ul / ms / ns, 0.0)[:, None] * w
    return bu + bw_norm, bu


def lact_head_bwd(q, k, v, eta, w1, w2, w3, dout, dw=None, *, chunk: int, order: int = 0,
                  rownorm: int = 1):
    """Gradients of L = sum dout * O + sum_i dw_i * W_i,final for one (batch, head).
    q [Tq, d]; k, v [Tkv, d]; eta [Tkv]; w1, w3 [hid, d]; w2 [d, hid]; dout [Tq, d];
    dw = (dw1, dw2, dw3) or None.  Returns (dq, dk, dv, deta, dw1, dw2, dw3) (the
    last three: gradients w.r.t. the initial weights)."""
    q, k, v, eta, dout = (np.asarray(a, dtype=np.float64) for a in (q, k, v, eta, dout))
    ws = [np.asarray(a, dtype=np.float64) for a in (w1, w2, w3)]
    Tkv, Tq = k.shape[0], q.shape[0]
    # forward, keeping the chunk-start weights and the chunk gradients
    starts, grads = [], []
    cs = list(range(0, Tkv, chunk))
    for c0 in cs:
        c1 = min(c0 + chunk, Tkv)
        d, _ = _chunk_grad(k[c0:c1], v[c0:c1], eta[c0:c1], *ws)
        starts.append([x.copy() for x in ws])
        grads.append(d)
        ws = [_step(ws[i], d[i], rownorm) for i in range(3)]
    lam = [np.zeros_like(x) for x in ws] if dw is None else [np.asarray(x, np.float64).copy()
                                                             for x in dw]
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    de = np.zeros_like(eta)
    if order == 1 and Tq > 0:
        bx, b1, b2, b3 = _apply_bwd(q, dout, *ws)
        dq[:] = bx
        lam = [lam[0] + b1, lam[1] + b2, lam[2] + b3]
    for ci in range(len(cs) - 1, -1, -1):
        c0 = cs[ci]
        c1 = min(c0 + chunk, Tkv)
        w = starts[ci]
        d = grads[ci]
        new_lam, gam = [], []
        for i in range(3):
            bw, bu = _step_bwd(w[i], d[i], lam[i], rownorm)
            new_lam.append(bw)
            gam.append(-bu)
        _, saved = _chunk_grad(k[c0:c1], v[c0:c1], eta[c0:c1], *w)
        b1, b2, b3, bk, bv, be = _chunk_grad_bwd(k[c0:c1], v[c0:c1], eta[c0:c1], *w, gam, saved)
        lam = [new_lam[0] + b1, new_lam[1] + b2, new_lam[2] + b3]
        dk[c0:c1] += bk
        dv[c0:c1] += bv
        de[c0:c1] += be
        if order == 0 and c0 < Tq:
            q1 = min(c1, Tq)
            bx, a1, a2, a3 = _apply_bwd(q[c0:q1], dout[c0:q1], *w)
            dq[c0:q1] = bx
            lam = [lam[0] + a1, lam[1] + a2, lam[2] + a3]
    return dq, dk, dv, de, lam[0], lam[1], lam[2]


def lact_swiglu_bwd(q, k, v, eta, w1, w2, w3, dout, dw=None, *, chunk: int, order: int = 0,
                    rownorm: int = 1):
    """All (batch, head) pairs: arrays with leading [B, H]; dw = (dw1, dw2, dw3) or None."""
    q = np.asarray(q)
    B, H = q.shape[:2]
    outs = None
    for b in range(B):
        for h in range(H):
            r = lact_head_bwd(q[b, h], k[b, h], v[b, h], eta[b, h], w1[b, h], w2[b, h], w3[b, h],
                              dout[b, h], None if dw is None else [x[b, h] for x in dw],
                              chunk=chunk, order=order, rownorm=rownorm)
            if outs is None:
                outs = [np.zeros((B, H) + x.shape) for x in r]
            for o, x in zip(outs, r):
                o[b, h] = x
    return tuple(outs)
