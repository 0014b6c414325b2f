"""Pins for the LaCT SwiGLU backward oracle (oracle/lact_backward.py; no GPU).

The backward differentiates the chunked LaCT forward ("LaCT: Test-Time
Training Done Right", sections 3.2-3.3 and 4: SwiGLU fast weight, negative
inner-product loss with per-token learning rate, summed chunk gradient,
gradient step, rows back to their pre-update norm, causal or update-then-apply
order) on the scalar L = sum(dO * O) + sum_i dW_i * W_i,final.  Its explicit
reverse mode (second derivatives of the SwiGLU MLP included) is checked
against three things it shares no code with:
  * central finite differences of the C token-loop forward oracle (itself
    pinned in test_oracle_pins.py),
  * torch's fp64 autograd through the same forward written with torch ops
    (differentiating through torch's own gradient: a double backward),
  * eta = 0, where nothing is learned: the weights never change, so the
    gradients are those of a plain SwiGLU MLP, written out here with element
    loops.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle.lact_backward import lact_head_bwd, lact_swiglu_bwd


def rel(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


def rand_case(seed, Tq, Tkv, d, hid, eta_scale=0.3):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((1, 1, Tq, d)) * 0.6
    k = rng.standard_normal((1, 1, Tkv, d)) * 0.6
    v = rng.standard_normal((1, 1, Tkv, d))
    eta = rng.uniform(0.2, 1.0, (1, 1, Tkv)) * eta_scale
    w1 = rng.standard_normal((1, 1, hid, d)) / np.sqrt(d)
    w2 = rng.standard_normal((1, 1, d, hid)) / np.sqrt(hid)
    w3 = rng.standard_normal((1, 1, hid, d)) / np.sqrt(d)
    do = rng.standard_normal((1, 1, Tq, d))
    dw = [rng.standard_normal(w.shape) for w in (w1, w2, w3)]
    return [q, k, v, eta, w1, w2, w3], do, dw


CASES = [  # Tq, Tkv, d, hid, chunk, order, rownorm
    (7, 7, 3, 5, 3, 0, 1), (7, 7, 3, 5, 7, 0, 0), (6, 6, 4, 6, 2, 0, 1),
    (4, 9, 3, 4, 4, 1, 1), (5, 8, 3, 5, 8, 1, 0),
]


@pytest.mark.parametrize("case", CASES)
def test_backward_matches_finite_differences(case):
    Tq, Tkv, d, hid, chunk, order, rownorm = case
    args, do, dw = rand_case(300 + Tkv + chunk + order, Tq, Tkv, d, hid)
    grads = lact_swiglu_bwd(*args, do, dw, chunk=chunk, order=order, rownorm=rownorm)

    def L(a):
        o, f1, f2, f3 = oracle.lact_swiglu(*a, chunk=chunk, loss=0, order=order, rownorm=rownorm)
        return float(np.sum(o * do) + np.sum(f1 * dw[0]) + np.sum(f2 * dw[1]) + np.sum(f3 * dw[2]))

    h = 1e-6
    for idx, g in enumerate(grads):
        base = args[idx]
        fd = np.zeros_like(base)
        it = np.nditer(base, flags=["multi_index"])
        for _ in it:
            mi = it.multi_index
            plus = [a.copy() for a in args]
            minus = [a.copy() for a in args]
            plus[idx][mi] += h
            minus[idx][mi] -= h
            fd[mi] = (L(plus) - L(minus)) / (2 * h)
        assert rel(g, fd) < 1e-6, ("q", "k", "v", "eta", "w1", "w2", "w3")[idx]


def _torch_forward(q, k, v, eta, w1, w2, w3, chunk, order, rownorm):
    """The forward in torch ops; each chunk's gradient by torch itself."""
    def f(x, a, b, c):
        return (torch.nn.functional.silu(x @ a.T) * (x @ c.T)) @ b.T
    ws = [w1, w2, w3]
    outs = []
    for c0 in range(0, k.shape[0], chunk):
        c1 = min(c0 + chunk, k.shape[0])
        if order == 0:
            outs.append(f(q[c0:c1], *ws))
        loss = -(eta[c0:c1, None] * f(k[c0:c1], *ws) * v[c0:c1]).sum()
        grads = torch.autograd.grad(loss, ws, create_graph=True)
        new = []
        for w, g in zip(ws, grads):
            u = w - g
            if rownorm:
                u = u * (torch.linalg.norm(w, dim=1) / torch.linalg.norm(u, dim=1))[:, None]
            new.append(u)
        ws = new
    if order == 1:
        outs = [f(q, *ws)]
    return torch.cat(outs, 0), ws


@pytest.mark.parametrize("case", CASES + [(12, 12, 6, 10, 5, 0, 1), (9, 13, 5, 7, 13, 1, 1)])
def test_backward_matches_torch_autograd(case):
    Tq, Tkv, d, hid, chunk, order, rownorm = case
    args, do, dw = rand_case(400 + Tkv + chunk + order, Tq, Tkv, d, hid)
    mine = lact_head_bwd(*[a[0, 0] for a in args], do[0, 0], [x[0, 0] for x in dw], chunk=chunk,
                         order=order, rownorm=rownorm)
    T = [torch.tensor(a[0, 0], dtype=torch.float64, requires_grad=True) for a in args]
    out, wf = _torch_forward(*T, chunk, order, rownorm)
    L = (out * torch.tensor(do[0, 0])).sum() + sum((w * torch.tensor(x[0, 0])).sum()
                                                   for w, x in zip(wf, dw))
    ref = torch.autograd.grad(L, T)
    for name, a, b in zip(("q", "k", "v", "eta", "w1", "w2", "w3"), mine, ref):
        assert rel(a, b.numpy()) < 1e-12, name


def test_eta_zero_is_a_plain_swiglu_mlp():
    """With eta = 0 the weights never move: dQ is the MLP's input gradient, the
    weight gradients are the MLP's weight gradients plus dW_final, and K, V,
    eta get exactly the gradient of the chunk gradient's eta-linear terms."""
    Tq = Tkv = 5
    d, hid = 3, 4
    args, do, dw = rand_case(77, Tq, Tkv, d, hid)
    args[3] = np.zeros_like(args[3])
    q, k, v, eta, w1, w2, w3 = [a[0, 0] for a in args]
    got = lact_head_bwd(q, k, v, eta, w1, w2, w3, do[0, 0], [x[0, 0] for x in dw], chunk=2,
                        order=0, rownorm=1)
    # the MLP's gradients with element loops
    sig = lambda z: 1.0 / (1.0 + np.exp(-z))
    dq = np.zeros_like(q)
    g1 = np.zeros_like(w1)
    g2 = np.zeros_like(w2)
    g3 = np.zeros_like(w3)
    for t in range(Tq):
        for j in range(hid):
            z1 = sum(w1[j, i] * q[t, i] for i in range(d))
            z3 = sum(w3[j, i] * q[t, i] for i in range(d))
            s = sig(z1)
            a = z1 * s
            up = sum(do[0, 0, t, o] * w2[o, j] for o in range(d))  # dL/dg_j
            for o in range(d):
                g2[o, j] += do[0, 0, t, o] * a * z3
            dz1 = up * z3 * s * (1.0 + z1 * (1.0 - s))
            dz3 = up * a
            for i in range(d):
                dq[t, i] += dz1 * w1[j, i] + dz3 * w3[j, i]
                g1[j, i] += dz1 * q[t, i]
                g3[j, i] += dz3 * q[t, i]
    assert rel(got[0], dq) < 1e-12
    assert rel(got[4], g1 + dw[0][0, 0]) < 1e-12
    assert rel(got[5], g2 + dw[1][0, 0]) < 1e-12
    assert rel(got[6], g3 + dw[2][0, 0]) < 1e-12
    # with eta = 0 only the eta-gradient can be nonzero among k, v, eta
    assert np.max(np.abs(got[1])) == 0.0 and np.max(np.abs(got[2])) == 0.0
    assert np.max(np.abs(got[3])) > 0.0


def test_no_upstream_weight_gradient_equals_zero_one():
    args, do, dw = rand_case(78, 6, 6, 3, 5)
    a = lact_swiglu_bwd(*args, do, None, chunk=3)
    b = lact_swiglu_bwd(*args, do, [np.zeros_like(x) for x in dw], chunk=3)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
