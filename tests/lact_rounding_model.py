"""A CPU model of where the bf16 LaCT kernels round, used to derive the
parity tolerances of the weight change and of the output change.

Test infrastructure only (numpy; no GPU code is run or imported).  It is not
the oracle: the oracle computes the method exactly in fp64.  This model
computes the same method ("LaCT: Test-Time Training Done Right", sections 3.2
and 3.3: SwiGLU fast weight, negative inner-product loss or MSE loss, summed
chunk gradient, gradient step, rows back to their pre-update L2 norm) but
rounds to bf16 at exactly the points where the kernels hand a value to a
bf16 matrix-core operand or to a bf16 output, and keeps everything else in
fp64 (the kernels accumulate in fp32, whose rounding is far below bf16's).
Rounding points modelled:

  * key forward and output gradient: the chunk-start weights enter as one
    bf16 rounding each (W1, W3, W2);
  * inner-product loss: dY = bf16(-eta * V);  MSE loss: dY = bf16(eta (f(K) - V))
    with f(K) from the applies (below);
  * epilogue of the key forward: G (times -eta for the inner-product loss),
    dH1 and dH3 each rounded once to bf16;
  * weight gradients: products of those bf16 operands (with K or V exact);
  * weights: fp32 masters (modelled exactly), step and row rescale;
  * applies: weights and G as bf16 hi/lo pairs (about 16 significant bits:
    modelled as hi + lo of the fp32 value), output rounded to bf16.

The difference between this model and the exact oracle is the error floor
that bf16 operands set for any implementation that rounds at these points.
The GPU tolerances are set with a margin over it (tests/parity.py).
"""
from __future__ import annotations

import numpy as np

from ttt_inputs import round_bf16


_EXACT = [False]   # True: every rounding below is the identity (the model is then the method)


def _r(x):
    if _EXACT[0]:
        return np.asarray(x, dtype=np.float64)
    return round_bf16(np.asarray(x, dtype=np.float32)).astype(np.float64)


def _f32(x):
    x = np.asarray(x)
    return x.astype(np.float64) if _EXACT[0] else x.astype(np.float32).astype(np.float64)


def _hilo(x):
    """hi + lo of an fp32 value as the kernels split it (hi = bf16(x), lo = bf16(x - hi))."""
    if _EXACT[0]:
        return np.asarray(x, dtype=np.float64)
    x = np.asarray(x, dtype=np.float32)
    hi = round_bf16(x)
    lo = round_bf16((x - hi).astype(np.float32))
    return hi.astype(np.float64) + lo.astype(np.float64)


def _sig(z):
    return 1.0 / (1.0 + np.exp(-z))


def _apply(x, w1, w2, w3):
    """f(x) rows with hi/lo weights and hi/lo G, output in fp64 (rounded by the caller)."""
    h1 = x @ _hilo(w1).T
    h3 = x @ _hilo(w3).T
    g = _hilo(h1 * _sig(h1) * h3)
    return g @ _hilo(w2).T


def _step(w, grad, rownorm):
    w = w.astype(np.float64)
    n0 = np.sqrt(np.sum(w * w, axis=1))
    x = w - grad
    if rownorm:
        n1 = np.sqrt(np.sum(x * x, axis=1))
        x = x * np.where(n1 > 0, n0 / np.where(n1 > 0, n1, 1.0), 1.0)[:, None]
    return x if _EXACT[0] else x.astype(np.float32)


def _newton_schulz_bf16(d, steps: int, tall: bool):
    """The kernels' cubic Newton-Schulz iteration: bf16 copies of the iterate and
    a bf16 Gram matrix as operands, fp32 iterate; step 0 runs on the unscaled
    direction with its norm taken from the Gram diagonal.  tall: the Gram is
    X^T X and the product X (X^T X) (W1, W3 layout); else X X^T and (X X^T) X."""
    x = d.astype(np.float64)
    for j in range(steps):
        xb = _r(x)
        gf = xb.T @ xb if tall else xb @ xb.T
        gram = _r(gf)
        prod = xb @ gram if tall else gram @ xb
        if j == 0:
            ss = float(np.trace(gf))
            if ss <= 0:
                return np.zeros_like(x)
            a, b = 1.5 / np.sqrt(ss), -0.5 / (np.sqrt(ss) * ss)
        else:
            a, b = 1.5, -0.5
        x = _f32(a * x + b * prod)
    return x


def lact_head_bf16_model(q, k, v, eta, w1, w2, w3, *, chunk: int, loss: int, order: int,
                         rownorm: int = 1, rule: int = 0, beta: float = 0.0, ns_steps: int = 5,
                         lr: float = 1.0, m=None, exact: bool = False):
    """One (batch, head) of the LaCT forward with the kernels' bf16 rounding points.
    Returns (out, w1, w2, w3) like oracle.dense.lact_head (out rounded to bf16).
    rule 1 (momentum) and 2 (Muon) update the momentum buffers m = [m1, m2, m3]
    in place when they keep one.  exact=True turns every rounding off (a check
    that the model computes the method itself)."""
    _EXACT[0] = bool(exact)
    try:
        return _model(q, k, v, eta, w1, w2, w3, chunk, loss, order, rownorm, rule, beta,
                      ns_steps, lr, m)
    finally:
        _EXACT[0] = False


def _model(q, k, v, eta, w1, w2, w3, chunk, loss, order, rownorm, rule, beta, ns_steps, lr, m):
    q, k, v = (np.asarray(a, dtype=np.float64) for a in (q, k, v))
    eta = np.asarray(eta, dtype=np.float64)
    w1, w2, w3 = (np.array(a, dtype=np.float64 if _EXACT[0] else np.float32)
                  for a in (w1, w2, w3))
    Tkv, Tq = k.shape[0], q.shape[0]
    out = np.zeros((Tq, q.shape[1]))
    use_m = rule == 1 or (rule == 2 and beta != 0.0)
    for c0 in range(0, Tkv, chunk):
        c1 = min(c0 + chunk, Tkv)
        if order == 0 and c0 < Tq:
            out[c0:min(c1, Tq)] = _apply(q[c0:min(c1, Tq)], w1, w2, w3)
        kc, vc, ec = k[c0:c1], v[c0:c1], eta[c0:c1]
        b1, b2, b3 = _r(w1), _r(w2), _r(w3)
        h1 = kc @ b1.T
        h3 = kc @ b3.T
        s = _sig(h1)
        a = h1 * s
        if loss == 1:
            dy = _r(ec[:, None] * (_r(_apply(kc, w1, w2, w3)) - vc))
            gmul = np.ones_like(ec)
        else:
            dy = _r(-ec[:, None] * vc)
            gmul = -ec
        dg = dy @ b2
        g = _r(a * h3 * gmul[:, None])          # G (carrying -eta for the inner product)
        dh3 = _r(dg * a)
        dh1 = _r(dg * h3 * (s * (1.0 + h1 * (1.0 - s))))
        grads = [dh1.T @ kc, (vc if loss == 0 else dy).T @ g, dh3.T @ kc]
        ws = [w1, w2, w3]
        for i in range(3):
            gi = _f32(grads[i])
            if use_m:
                m[i][:] = _f32(beta * m[i] + gi)
                gi = m[i].astype(np.float64)
            if rule == 2:
                gi = lr * _newton_schulz_bf16(gi, ns_steps, tall=(i != 1))
            ws[i] = _step(ws[i], gi, rownorm)
        w1, w2, w3 = ws
    if order == 1:
        out[:] = _apply(q, w1, w2, w3)
    return _r(out), np.asarray(w1, np.float64), np.asarray(w2, np.float64), np.asarray(w3, np.float64)


def delta_errors(got, ref, base):
    """(max |got - ref| / RMS(ref - base),
        max(|got - ref| - 2^-8 |ref|) / RMS(ref - base))"""
    got, ref, base = (np.asarray(a, dtype=np.float64) for a in (got, ref, base))
    drms = float(np.sqrt(np.mean((ref - base) ** 2)))
    d = np.abs(got - ref)
    return float(d.max() / drms), float(np.max(d - np.abs(ref) * 2.0 ** -8) / drms)
