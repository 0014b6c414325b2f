"""Pins for the TTT-Linear backward oracle (no GPU).

The backward differentiates the causal token-by-token forward of "Test-Time
Training (TTT)" ("TTT definition", examples 1 and 2, "Mini-batch gradient
descent").  It is checked against central finite differences of the forward
oracle (the C token loop, pinned in test_oracle_pins.py) on the scalar
L = sum(dy * y) + sum(dW * W_final), against torch's fp64 autograd of the
same steps written with torch ops, and against the closed-form gradients of
causal linear attention for the inner-product loss from a zero state.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle.backward import ttt_linear_bwd


def rel(a, b):
    a, b = np.asarray(a), np.asarray(b)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


def rand_case(seed, B=1, H=2, T=7, d=3):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, H, T, d)) / np.sqrt(d)
    k = rng.standard_normal((B, H, T, d)) / np.sqrt(d)
    v = rng.standard_normal((B, H, T, d))
    eta = rng.uniform(0.05, 0.4, (B, H, T))
    w0 = rng.standard_normal((B, H, d, d)) / np.sqrt(d)
    dy = rng.standard_normal((B, H, T, d))
    dwf = rng.standard_normal((B, H, d, d))
    return q, k, v, eta, w0, dy, dwf


@pytest.mark.parametrize("loss", [0, 1])
@pytest.mark.parametrize("chunk", [1, 3, 7, 10])
def test_backward_matches_finite_differences(loss, chunk):
    q, k, v, eta, w0, dy, dwf = rand_case(100 + chunk + loss)
    grads = ttt_linear_bwd(q, k, v, eta, w0, dy, dwf, chunk=chunk, loss=loss)

    def L(args):
        y, wf = oracle.ttt_linear(*args, chunk=chunk, loss=loss)
        return float(np.sum(y * dy) + np.sum(wf * dwf))

    base = [q, k, v, eta, w0]
    h = 1e-6
    for idx, g in enumerate(grads):
        fd = np.zeros_like(base[idx])
        it = np.nditer(base[idx], flags=["multi_index"])
        for _ in it:
            mi = it.multi_index
            plus = [a.copy() for a in base]
            minus = [a.copy() for a in base]
            plus[idx][mi] += h
            minus[idx][mi] -= h
            fd[mi] = (L(plus) - L(minus)) / (2 * h)
        assert rel(g, fd) < 1e-7, ("q", "k", "v", "eta", "w0")[idx]


@pytest.mark.parametrize("loss", [0, 1])
def test_backward_matches_torch_autograd(loss):
    """The same steps in torch ops, differentiated by torch's fp64 autograd."""
    chunk = 4
    q, k, v, eta, w0, dy, dwf = rand_case(200 + loss, T=11, d=5)
    ts = [torch.tensor(a, requires_grad=True) for a in (q, k, v, eta, w0)]
    tq, tk, tv, te, tw = ts
    T = q.shape[2]
    ys = []
    W = tw
    for c0 in range(0, T, chunk):
        Wc = W
        for t in range(c0, min(c0 + chunk, T)):
            kt = tk[:, :, t, :]
            r = torch.einsum("bhi,bhij->bhj", kt, Wc) - tv[:, :, t, :] if loss else -tv[:, :, t, :]
            W = W - te[:, :, t, None, None] * kt[..., :, None] * r[..., None, :]
            ys.append(torch.einsum("bhi,bhij->bhj", tq[:, :, t, :], W))
    y = torch.stack(ys, dim=2)
    Ltot = (y * torch.tensor(dy)).sum() + (W * torch.tensor(dwf)).sum()
    Ltot.backward()
    grads = ttt_linear_bwd(q, k, v, eta, w0, dy, dwf, chunk=chunk, loss=loss)
    for g, t in zip(grads, ts):
        assert rel(g, t.grad.numpy()) < 1e-12


def test_dot_zero_state_closed_form():
    """Inner-product loss from W0 = 0 is causal linear attention,
    y_t = sum_{i<=t} eta_i (q_t . k_i) v_i, whose gradients are
    dq_t = sum_{i<=t} eta_i (dy_t . v_i) k_i,  dk_i = eta_i sum_{t>=i} (dy_t . v_i) q_t,
    dv_i = eta_i sum_{t>=i} (q_t . k_i) dy_t,  deta_i = sum_{t>=i} (q_t . k_i)(dy_t . v_i)
    (chunk size does not matter for this loss)."""
    q, k, v, eta, w0, dy, _ = rand_case(300, T=9, d=4)
    w0 = np.zeros_like(w0)
    dq, dk, dv, de, dw0 = ttt_linear_bwd(q, k, v, eta, w0, dy, None, chunk=4, loss=0)
    T = q.shape[2]
    for b in range(q.shape[0]):
        for h in range(q.shape[1]):
            Q, K, V, E, DY = q[b, h], k[b, h], v[b, h], eta[b, h], dy[b, h]
            for t in range(T):
                ref = sum(E[i] * np.dot(DY[t], V[i]) * K[i] for i in range(t + 1))
                assert rel(dq[b, h, t], ref) < 1e-12
            for i in range(T):
                assert rel(dk[b, h, i], E[i] * sum(np.dot(DY[t], V[i]) * Q[t] for t in range(i, T))) < 1e-12
                assert rel(dv[b, h, i], E[i] * sum(np.dot(Q[t], K[i]) * DY[t] for t in range(i, T))) < 1e-12
                assert abs(de[b, h, i] - sum(np.dot(Q[t], K[i]) * np.dot(DY[t], V[i])
                                             for t in range(i, T))) < 1e-12
    # dW0 = sum_t q_t^T dy_t
    assert rel(dw0[0, 0], q[0, 0].T @ dy[0, 0]) < 1e-12


@pytest.mark.parametrize("loss", [0, 1])
@pytest.mark.parametrize("chunk", [1, 4, 20])
def test_noncausal_backward_matches_finite_differences(loss, chunk):
    """Update over all key/value chunks, then every query reads the final state."""
    rng = np.random.default_rng(400 + chunk + loss)
    B, H, Tq, Tkv, d = 1, 2, 5, 9, 3
    q = rng.standard_normal((B, H, Tq, d)) / np.sqrt(d)
    k = rng.standard_normal((B, H, Tkv, d)) / np.sqrt(d)
    v = rng.standard_normal((B, H, Tkv, d))
    eta = rng.uniform(0.05, 0.4, (B, H, Tkv))
    w0 = rng.standard_normal((B, H, d, d)) / np.sqrt(d)
    dy = rng.standard_normal((B, H, Tq, d))
    dwf = rng.standard_normal((B, H, d, d))
    grads = ttt_linear_bwd(q, k, v, eta, w0, dy, dwf, chunk=chunk, loss=loss, order=1)

    def L(args):
        y, wf = oracle.ttt_linear(*args, chunk=chunk, loss=loss, order=oracle.NONCAUSAL)
        return float(np.sum(y * dy) + np.sum(wf * dwf))

    base = [q, k, v, eta, w0]
    h = 1e-6
    for idx, g in enumerate(grads):
        fd = np.zeros_like(base[idx])
        it = np.nditer(base[idx], flags=["multi_index"])
        for _ in it:
            mi = it.multi_index
            plus = [a.copy() for a in base]
            minus = [a.copy() for a in base]
            plus[idx][mi] += h
            minus[idx][mi] -= h
            fd[mi] = (L(plus) - L(minus)) / (2 * h)
        assert rel(g, fd) < 1e-7, ("q", "k", "v", "eta", "w0")[idx]
