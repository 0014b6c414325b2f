"""Pins for the single-token decode oracle (no GPU).

The decode step is the per-token rule of "Test-Time Training (TTT)": the state
carried from token to token takes one gradient step per token ("TTT
definition"), with the gradients of examples 1 and 2, and, for chunked
decoding, every gradient of a chunk taken at the chunk-start state
("Mini-batch gradient descent").  Each test checks ``oracle.decode`` against
something other than its own formula: causal linear attention by brute force,
the delta rule's write property, invariants, central finite differences, and
the token-by-token C oracle (independent code, pinned in test_oracle_pins.py)
over every chunk size on a ragged sequence.
"""
import numpy as np
import pytest

import oracle
from oracle import decode


def rel(a, b):
    a, b = np.asarray(a), np.asarray(b)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


def rand_seq(rng, B, H, T, d):
    q = rng.standard_normal((B, H, T, d)) / np.sqrt(d)
    k = rng.standard_normal((B, H, T, d)) / np.sqrt(d)
    v = rng.standard_normal((B, H, T, d))
    eta = rng.uniform(0.02, 0.4, (B, H, T))
    w0 = rng.standard_normal((B, H, d, d)) / np.sqrt(d)
    return q, k, v, eta, w0


def test_dot_decode_is_causal_linear_attention():
    """Inner-product loss: decoding token by token is causal linear attention,
    y_t = q_t W0 + sum_{i<=t} eta_i (q_t . k_i) v_i (brute force over i)."""
    rng = np.random.default_rng(21)
    q, k, v, eta, w0 = rand_seq(rng, 2, 3, 19, 8)
    y, wf = decode.ttt_linear_decode_sequence(q, k, v, eta, w0, loss=decode.LOSS_DOT)
    ref = np.zeros_like(y)
    for b in range(2):
        for h in range(3):
            for t in range(19):
                acc = q[b, h, t] @ w0[b, h]
                for i in range(t + 1):
                    acc = acc + eta[b, h, i] * np.dot(q[b, h, t], k[b, h, i]) * v[b, h, i]
                ref[b, h, t] = acc
    assert rel(y, ref) < 1e-12


def test_mse_decode_writes_value_at_key():
    """MSE loss (the delta rule): with eta = 1/||k||^2 one step stores v at key k,
    k W' = v exactly, and leaves every direction orthogonal to k unchanged."""
    rng = np.random.default_rng(22)
    B, H, d = 2, 2, 12
    q = rng.standard_normal((B, H, d))
    k = rng.standard_normal((B, H, d))
    v = rng.standard_normal((B, H, d))
    w = rng.standard_normal((B, H, d, d))
    eta = 1.0 / np.sum(k * k, axis=-1)
    y, wn, _ = decode.ttt_linear_decode(q, k, v, eta, w, loss=decode.LOSS_MSE)
    for b in range(B):
        for h in range(H):
            assert rel(k[b, h] @ wn[b, h], v[b, h]) < 1e-12
            x = rng.standard_normal(d)
            x -= np.dot(x, k[b, h]) / np.dot(k[b, h], k[b, h]) * k[b, h]
            assert rel(x @ wn[b, h], x @ w[b, h]) < 1e-10
            assert rel(y[b, h], q[b, h] @ wn[b, h]) < 1e-12


@pytest.mark.parametrize("loss", [decode.LOSS_DOT, decode.LOSS_MSE])
def test_decode_step_is_minus_eta_fd_gradient(loss):
    """W' = W - eta * grad, the gradient of the token's loss at the anchor state,
    checked against central finite differences of the loss written out here."""
    rng = np.random.default_rng(23)
    d = 6
    q, k, v = (rng.standard_normal((1, 1, d)) for _ in range(3))
    w = rng.standard_normal((1, 1, d, d))
    anchor = rng.standard_normal((1, 1, d, d))
    eta = np.array([[0.37]])

    def lossf(W):
        p = k[0, 0] @ W
        if loss == decode.LOSS_MSE:
            return 0.5 * np.sum((p - v[0, 0]) ** 2)
        return -np.dot(p, v[0, 0])

    fd = np.zeros((d, d))
    hstep = 1e-6
    for i in range(d):
        for j in range(d):
            e = np.zeros((d, d))
            e[i, j] = hstep
            fd[i, j] = (lossf(anchor[0, 0] + e) - lossf(anchor[0, 0] - e)) / (2 * hstep)
    _, wn, an = decode.ttt_linear_decode(q, k, v, eta, w, anchor, loss=loss)
    assert rel(wn[0, 0], w[0, 0] - 0.37 * fd) < 1e-8
    assert np.array_equal(an, anchor)          # not the chunk's last token: anchor kept


@pytest.mark.parametrize("loss", [decode.LOSS_DOT, decode.LOSS_MSE])
@pytest.mark.parametrize("chunk", [1, 2, 3, 16, 37, 40])
def test_decode_sequence_matches_token_loop_oracle(loss, chunk):
    """Decoding a ragged 37-token sequence one token at a time, with the anchor
    moved at every chunk's end, equals the chunked forward of the C token loop
    for every chunk size (1 = the recurrent rule; 40 > T = one chunk)."""
    rng = np.random.default_rng(24 + chunk)
    q, k, v, eta, w0 = rand_seq(rng, 2, 2, 37, 8)
    y, wf = decode.ttt_linear_decode_sequence(q, k, v, eta, w0, loss=loss, chunk=chunk)
    ref_y, ref_w = oracle.ttt_linear(q, k, v, eta, w0, chunk=chunk, loss=loss)
    assert rel(y, ref_y) < 1e-11
    assert rel(wf, ref_w) < 1e-11


def test_decode_anchor_update_moves_anchor():
    rng = np.random.default_rng(25)
    d = 5
    q, k, v = (rng.standard_normal((1, 1, d)) for _ in range(3))
    w = rng.standard_normal((1, 1, d, d))
    anchor = rng.standard_normal((1, 1, d, d))
    _, wn, an = decode.ttt_linear_decode(q, k, v, np.array([[0.2]]), w, anchor,
                                         loss=decode.LOSS_MSE, anchor_update=True)
    assert np.array_equal(an, wn)
    assert not np.array_equal(wn, w)
