"""LaCT SwiGLU oracle with each chunk's token sums done by numpy fp64 matmuls.

Test infrastructure, like the rest of ``oracle/``.  Same definitions as the
token loop in ``ttt_oracle.c`` ("LaCT: Test-Time Training Done Right",
sections 3.2-3.3 and 4): per chunk, the summed gradient of
sum_t eta_t L_t at the chunk-start weights, a step (plain gradient descent,
momentum, or Muon: the cubic Newton-Schulz iteration for the polar factor of
the momentum, section 3.3 naming the three rules), then each row back to its
pre-update L2 norm.  The only difference is that a
sum over a chunk's tokens (sum_t dy_t g_t^T and the like) is written as one
matrix product instead of a Python-level loop, which makes the full-size
workloads (chunks of 2048 and 65536 tokens) affordable.  It is pinned against
the token loop in the tests.

Rows are tokens: X [n, d]; H1 = X W1^T, H3 = X W3^T, G = silu(H1) * H3,
Y = G W2^T.
"""
from __future__ import annotations

import numpy as np


def _sigmoid(z):
    return 1.0 / (1.0 + np.exp(-z))


def swiglu_apply(x, w1, w2, w3):
    """f applied to every row of x [n, d]; w1, w3 [hid, d], w2 [d, hid]."""
    h1 = x @ w1.T
    h3 = x @ w3.T
    return (h1 * _sigmoid(h1) * h3) @ w2.T


def chunk_grad(x, v, eta, w1, w2, w3, loss: int):
    """Gradients (G1, G2, G3) of sum_t eta_t L_t over the rows of x at (w1, w2, w3)."""
    h1 = x @ w1.T
    h3 = x @ w3.T
    s = _sigmoid(h1)
    a = h1 * s
    g = a * h3
    if loss == 1:
        dy = eta[:, None] * (g @ w2.T - v)
    else:
        dy = -eta[:, None] * v
    g2 = dy.T @ g
    dg = dy @ w2
    dh3 = dg * a
    dh1 = dg * h3 * (s * (1.0 + h1 * (1.0 - s)))
    g1 = dh1.T @ x
    g3 = dh3.T @ x
    return g1, g2, g3


def _rownorm_step(w, g, rownorm: int):
    n_before = np.sqrt(np.sum(w * w, axis=1))
    w = w - g
    if rownorm:
        n_after = np.sqrt(np.sum(w * w, axis=1))
        f = np.where(n_after == 0.0, 1.0, n_before / np.where(n_after == 0.0, 1.0, n_after))
        w = w * f[:, None]
    return w


def newton_schulz(m, steps: int):
    """k steps of the cubic Newton-Schulz iteration for the orthogonal polar
    factor from X_0 = m / ||m||_F: X <- 1.5 X - 0.5 X (X^T X); zero maps to zero."""
    m = np.asarray(m, dtype=np.float64)
    nrm = np.sqrt(np.sum(m * m))
    if nrm == 0.0:
        return np.zeros_like(m)
    x = m / nrm
    for _ in range(steps):
        x = 1.5 * x - 0.5 * (x @ (x.T @ x))
    return x


def _direction(g, mbuf, rule: int, beta: float, ns_steps: int, lr: float):
    """Step direction for gradient descent (0), momentum (1) or Muon (2); updates
    the momentum buffer in place where the rule keeps one."""
    if rule == 0:
        return g
    if mbuf is not None:
        mbuf *= beta
        mbuf += g
        g = mbuf.copy()
    if rule == 2:
        g = lr * newton_schulz(g, ns_steps)
    return g


def lact_head(q, k, v, eta, w1, w2, w3, *, chunk: int, loss: int = 0, order: int = 0,
              rownorm: int = 1, q_rows=None, rule: int = 0, beta: float = 0.0,
              ns_steps: int = 5, lr: float = 1.0, m=None):
    """One (batch, head).  Returns (out_rows, w1, w2, w3) where out_rows are the
    outputs of the query rows listed in ``q_rows`` (all rows when None).  With
    rule 1 (momentum) or 2 (Muon), ``m`` = [m1, m2, m3] momentum buffers are
    updated in place (required unless rule is 0, or 2 with beta == 0)."""
    q, k, v, eta = (np.asarray(a, dtype=np.float64) for a in (q, k, v, eta))
    w1, w2, w3 = (np.array(a, dtype=np.float64) for a in (w1, w2, w3))
    Tkv = k.shape[0]
    Tq = q.shape[0]
    rows = np.arange(Tq) if q_rows is None else np.asarray(q_rows)
    out = np.zeros((len(rows), q.shape[1]))
    for c0 in range(0, Tkv, chunk):
        c1 = min(c0 + chunk, Tkv)
        if order == 0:
            sel = np.nonzero((rows >= c0) & (rows < c1))[0]
            if len(sel):
                out[sel] = swiglu_apply(q[rows[sel]], w1, w2, w3)
        g1, g2, g3 = chunk_grad(k[c0:c1], v[c0:c1], eta[c0:c1], w1, w2, w3, loss)
        use_m = rule == 1 or (rule == 2 and beta != 0.0)
        g1, g2, g3 = (_direction(g, m[i] if use_m else None, rule, beta, ns_steps, lr)
                      for i, g in enumerate((g1, g2, g3)))
        w1 = _rownorm_step(w1, g1, rownorm)
        w2 = _rownorm_step(w2, g2, rownorm)
        w3 = _rownorm_step(w3, g3, rownorm)
    if order == 1:
        out[:] = swiglu_apply(q[rows], w1, w2, w3)
    return out, w1, w2, w3
