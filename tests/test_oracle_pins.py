"""Pins for the CPU oracle (no GPU).

Each test checks the oracle against something other than itself: a closed form
the pages state, a textbook recurrence, dense matrix algebra written here,
central finite differences, an invariant, or brute force over every chunk size
on tiny inputs.  The sources are the pages' sections:

* "Test-Time Training (TTT)" summary -- "Linear Attention" (S_t = S_{t-1} +
  k_t^T v_t, y_t = q_t S_t), "TTT definition", example 1 (inner-product loss ->
  linear-attention update), example 2 (MSE loss -> delta rule with forgetting
  and inserting terms), "TTT-Linear", "Mini-batch gradient descent".
* "LaCT: Test-Time Training Done Right" -- sections 3.2 (SwiGLU fast weight,
  negative inner-product loss, per-token lr, summed chunk gradient), 3.3 (GD +
  L2 normalisation), 4 (update/apply orders).
"""
import json
import os

import numpy as np
import pytest

import oracle
from oracle import dense

RTOL = 1e-12
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rel(a, b):
    a, b = np.asarray(a), np.asarray(b)
    den = max(np.max(np.abs(b)), 1e-300)
    return float(np.max(np.abs(a - b)) / den)


def rand_linear(rng, B, H, T, d, Tq=None, w0="normal"):
    Tq = T if Tq is None else Tq
    q = rng.standard_normal((B, H, Tq, d)) / np.sqrt(d)
    k = rng.standard_normal((B, H, T, d)) / np.sqrt(d)
    v = rng.standard_normal((B, H, T, d))
    eta = rng.uniform(0.01, 0.3, (B, H, T))
    if w0 == "normal":
        w = rng.standard_normal((B, H, d, d)) / np.sqrt(d)
    else:
        w = np.zeros((B, H, d, d))
    return q, k, v, eta, w


# --------------------------------------------------------------------------
# TTT-Linear, inner-product loss == causal linear attention
# --------------------------------------------------------------------------
@pytest.mark.parametrize("chunk", [1, 3, 16, 37, 64])
def test_dot_equals_linear_attention_recurrence(chunk):
    """Example 1: with L = -(kW).v the update is W += eta k^T v, i.e. the
    linear-attention state S_t = S_{t-1} + eta_t k_t^T v_t read as y_t = q_t S_t."""
    rng = np.random.default_rng(11)
    q, k, v, eta, w0 = rand_linear(rng, 2, 2, 37, 8)
    out, wf = oracle.ttt_linear(q, k, v, eta, w0, chunk=chunk, loss=oracle.LOSS_DOT)
    ref = np.zeros_like(out)
    for b in range(2):
        for h in range(2):
            S = w0[b, h].copy()
            for t in range(37):
                S = S + eta[b, h, t] * np.outer(k[b, h, t], v[b, h, t])
                ref[b, h, t] = q[b, h, t] @ S
            assert rel(wf[b, h], S) < RTOL
    assert rel(out, ref) < RTOL


def test_dot_config_form_is_scaled_causal_linear_attention():
    """eta = 0.1 everywhere and W0 = 0: y = 0.1 * (Q K^T masked to i <= t) V."""
    rng = np.random.default_rng(12)
    T, d = 48, 16
    q, k, v, _, _ = rand_linear(rng, 1, 1, T, d)
    eta = np.full((1, 1, T), 0.1)
    out, _ = oracle.ttt_linear(q, k, v, eta, np.zeros((1, 1, d, d)), chunk=16,
                               loss=oracle.LOSS_DOT)
    A = np.tril(q[0, 0] @ k[0, 0].T)
    assert rel(out[0, 0], 0.1 * (A @ v[0, 0])) < RTOL


def test_dot_independent_of_chunk_size():
    rng = np.random.default_rng(13)
    q, k, v, eta, w0 = rand_linear(rng, 1, 3, 50, 6)
    base = oracle.ttt_linear(q, k, v, eta, w0, chunk=1, loss=oracle.LOSS_DOT)
    for b in (2, 7, 16, 50, 99):
        o, w = oracle.ttt_linear(q, k, v, eta, w0, chunk=b, loss=oracle.LOSS_DOT)
        assert rel(o, base[0]) < RTOL and rel(w, base[1]) < RTOL


# --------------------------------------------------------------------------
# TTT-Linear, MSE loss
# --------------------------------------------------------------------------
def test_mse_chunk1_equals_delta_rule():
    """Example 2: W_t = W_{t-1} - eta_t k_t^T (k_t W_{t-1} - v_t), y_t = q_t W_t."""
    rng = np.random.default_rng(21)
    q, k, v, eta, w0 = rand_linear(rng, 2, 2, 40, 8)
    out, wf = oracle.ttt_linear(q, k, v, eta, w0, chunk=1, loss=oracle.LOSS_MSE)
    for b in range(2):
        for h in range(2):
            W = w0[b, h].copy()
            for t in range(40):
                kt, vt = k[b, h, t], v[b, h, t]
                # forgetting term eta k^T k W and inserting term eta k^T v
                W = W - eta[b, h, t] * np.outer(kt, kt) @ W + eta[b, h, t] * np.outer(kt, vt)
                assert rel(out[b, h, t], q[b, h, t] @ W) < 1e-11
            assert rel(wf[b, h], W) < RTOL


def dual_form(q, k, v, eta, w0, chunk, loss):
    """Chunk recursion in matrix form, written independently of the oracle:
    W_{c+1} = W_c - K_c^T H_c R_c with R_c = K_c W_c - V_c (MSE) or -V_c (DOT),
    O_c = Q_c W_c + ((Q_c K_c^T) * M_incl * eta^T) U_c with U_c = -R_c."""
    T, d = k.shape
    W = w0.copy()
    O = np.zeros((q.shape[0], d))
    for c0 in range(0, T, chunk):
        c1 = min(c0 + chunk, T)
        K, V, Q, e = k[c0:c1], v[c0:c1], q[c0:c1], eta[c0:c1]
        U = (V - K @ W) if loss == 1 else V
        A = np.tril(Q @ K.T) * e[None, :]
        O[c0:c1] = Q @ W + A @ U
        W = W + K.T @ (e[:, None] * U)
    return O, W


def test_mse_single_chunk_dense_algebra():
    """One chunk (b >= T): y = Q W0 + (Q K^T * M * eta)(V - K W0),
    W_T = W0 + K^T diag(eta) (V - K W0)."""
    rng = np.random.default_rng(22)
    T, d = 24, 8
    q, k, v, eta, w0 = rand_linear(rng, 1, 1, T, d)
    out, wf = oracle.ttt_linear(q, k, v, eta, w0, chunk=32, loss=oracle.LOSS_MSE)
    Q, K, V, e, W0 = q[0, 0], k[0, 0], v[0, 0], eta[0, 0], w0[0, 0]
    U = V - K @ W0
    y = Q @ W0 + (np.tril(Q @ K.T) * e[None, :]) @ U
    W = W0 + K.T @ np.diag(e) @ U
    assert rel(out[0, 0], y) < RTOL
    assert rel(wf[0, 0], W) < RTOL


@pytest.mark.parametrize("chunk", [2, 5, 16, 33])
@pytest.mark.parametrize("loss", [0, 1])
def test_general_chunk_matches_dual_form(chunk, loss):
    rng = np.random.default_rng(23 + chunk)
    q, k, v, eta, w0 = rand_linear(rng, 1, 2, 70, 8)
    out, wf = oracle.ttt_linear(q, k, v, eta, w0, chunk=chunk, loss=loss)
    for h in range(2):
        O, W = dual_form(q[0, h], k[0, h], v[0, h], eta[0, h], w0[0, h], chunk, loss)
        assert rel(out[0, h], O) < 1e-10
        assert rel(wf[0, h], W) < 1e-10


def test_brute_force_every_chunk_size_tiny():
    """All b in 1..T, T <= 8, d <= 4, both losses: token loop vs dual form."""
    rng = np.random.default_rng(24)
    for T in range(1, 9):
        for d in (1, 2, 4):
            q, k, v, eta, w0 = rand_linear(rng, 1, 1, T, d)
            for loss in (0, 1):
                for b in range(1, T + 1):
                    out, wf = oracle.ttt_linear(q, k, v, eta, w0, chunk=b, loss=loss)
                    O, W = dual_form(q[0, 0], k[0, 0], v[0, 0], eta[0, 0], w0[0, 0], b, loss)
                    assert rel(out[0, 0], O) < 1e-11, (T, d, loss, b)
                    assert rel(wf[0, 0], W) < 1e-11, (T, d, loss, b)


@pytest.mark.parametrize("loss", [0, 1])
def test_update_is_minus_eta_times_fd_gradient(loss):
    """One chunk: W_final - W0 = -grad_W sum_t eta_t L_t(W0), with L the
    page's loss (MSE 1/2||kW-v||^2 or -(kW).v), by central differences."""
    rng = np.random.default_rng(25)
    T, d = 5, 4
    q, k, v, eta, w0 = rand_linear(rng, 1, 1, T, d)
    _, wf = oracle.ttt_linear(q, k, v, eta, w0, chunk=T, loss=loss)
    K, V, e = k[0, 0], v[0, 0], eta[0, 0]

    def total(W):
        P = K @ W
        if loss == 1:
            return float(np.sum(e * 0.5 * np.sum((P - V) ** 2, axis=1)))
        return float(np.sum(e * -np.sum(P * V, axis=1)))

    W0 = w0[0, 0]
    grad = np.zeros_like(W0)
    hstep = 1e-5
    for i in range(d):
        for j in range(d):
            Wp, Wm = W0.copy(), W0.copy()
            Wp[i, j] += hstep
            Wm[i, j] -= hstep
            grad[i, j] = (total(Wp) - total(Wm)) / (2 * hstep)
    assert rel(wf[0, 0] - W0, -grad) < 1e-6


@pytest.mark.parametrize("loss", [0, 1])
def test_eta_zero_is_plain_apply(loss):
    rng = np.random.default_rng(26)
    q, k, v, eta, w0 = rand_linear(rng, 2, 1, 20, 8)
    out, wf = oracle.ttt_linear(q, k, v, 0 * eta, w0, chunk=4, loss=loss)
    assert np.array_equal(wf, w0)
    assert rel(out, np.einsum("bhti,bhij->bhtj", q, w0)) < RTOL


@pytest.mark.parametrize("loss", [0, 1])
def test_state_carry_resume(loss):
    rng = np.random.default_rng(27)
    q, k, v, eta, w0 = rand_linear(rng, 1, 2, 64, 8)
    full_o, full_w = oracle.ttt_linear(q, k, v, eta, w0, chunk=8, loss=loss)
    T1 = 24
    o1, w1 = oracle.ttt_linear(q[:, :, :T1], k[:, :, :T1], v[:, :, :T1], eta[:, :, :T1], w0,
                               chunk=8, loss=loss)
    o2, w2 = oracle.ttt_linear(q[:, :, T1:], k[:, :, T1:], v[:, :, T1:], eta[:, :, T1:], w1,
                               chunk=8, loss=loss)
    assert rel(np.concatenate([o1, o2], axis=2), full_o) < RTOL
    assert rel(w2, full_w) < RTOL


def test_head_isolation():
    rng = np.random.default_rng(28)
    q, k, v, eta, w0 = rand_linear(rng, 2, 3, 32, 8)
    base_o, base_w = oracle.ttt_linear(q, k, v, eta, w0, chunk=8, loss=1)
    k2 = k.copy()
    k2[1, 2] += 0.5
    o, w = oracle.ttt_linear(q, k2, v, eta, w0, chunk=8, loss=1)
    mask = np.ones((2, 3), bool)
    mask[1, 2] = False
    assert np.array_equal(o[mask], base_o[mask]) and np.array_equal(w[mask], base_w[mask])
    assert not np.array_equal(o[1, 2], base_o[1, 2])


@pytest.mark.parametrize("loss", [0, 1])
def test_noncausal_reads_final_state(loss):
    rng = np.random.default_rng(29)
    q, k, v, eta, w0 = rand_linear(rng, 1, 2, 40, 8, Tq=13)
    out, wf = oracle.ttt_linear(q, k, v, eta, w0, chunk=16, loss=loss, order=oracle.NONCAUSAL)
    for h in range(2):
        _, W = dual_form(k[0, h], k[0, h], v[0, h], eta[0, h], w0[0, h], 16, loss)
        assert rel(wf[0, h], W) < 1e-11
        assert rel(out[0, h], q[0, h] @ W) < 1e-11


def test_handworked_golden_linear():
    """Exact values worked by hand from the update and query rules (file cites them)."""
    with open(os.path.join(GOLDEN, "hand_worked.json")) as f:
        g = json.load(f)
    for case in g["ttt_linear"]:
        arr = lambda n: np.array(case[n], dtype=np.float64)[None, None]
        out, wf = oracle.ttt_linear(arr("q"), arr("k"), arr("v"), arr("eta"), arr("w0"),
                                    chunk=case["chunk"], loss=case["loss"])
        np.testing.assert_allclose(out[0, 0], np.array(case["out"]), rtol=0, atol=1e-14)
        np.testing.assert_allclose(wf[0, 0], np.array(case["w_final"]), rtol=0, atol=1e-14)


def test_oracle_rejects_bad_arguments():
    z = np.zeros((1, 1, 4, 2))
    with pytest.raises(ValueError):
        oracle.ttt_linear(z, z, z, np.zeros((1, 1, 4)), np.zeros((1, 1, 2, 2)), chunk=0, loss=0)
    with pytest.raises(ValueError):
        oracle.ttt_linear(z, z, z, np.zeros((1, 1, 4)), np.zeros((1, 1, 2, 2)), chunk=2, loss=3)


# --------------------------------------------------------------------------
# LaCT SwiGLU
# --------------------------------------------------------------------------
def swiglu_ref(x, w1, w2, w3):
    """f(x) = W2 (silu(W1 x) * (W3 x)) for one column vector x, element loops."""
    hid, d = w1.shape
    y = np.zeros(w2.shape[0])
    for r in range(hid):
        h1 = sum(w1[r, i] * x[i] for i in range(d))
        h3 = sum(w3[r, i] * x[i] for i in range(d))
        a = h1 / (1.0 + np.exp(-h1))
        y += w2[:, r] * (a * h3)
    return y


def rand_lact(rng, B, H, T, d, hid, Tq=None):
    Tq = T if Tq is None else Tq
    q = rng.standard_normal((B, H, Tq, d))
    k = rng.standard_normal((B, H, T, d))
    v = rng.standard_normal((B, H, T, d))
    eta = rng.uniform(0.05, 0.5, (B, H, T))
    w1 = rng.standard_normal((B, H, hid, d)) / np.sqrt(d)
    w2 = rng.standard_normal((B, H, d, hid)) / np.sqrt(hid)
    w3 = rng.standard_normal((B, H, hid, d)) / np.sqrt(d)
    return q, k, v, eta, w1, w2, w3


def test_lact_eta_zero_is_swiglu_mlp():
    rng = np.random.default_rng(31)
    q, k, v, eta, w1, w2, w3 = rand_lact(rng, 1, 2, 9, 4, 8)
    out, f1, f2, f3 = oracle.lact_swiglu(q, k, v, 0 * eta, w1, w2, w3, chunk=4)
    assert np.array_equal(f1, w1) and np.array_equal(f2, w2) and np.array_equal(f3, w3)
    for h in range(2):
        for t in range(9):
            assert rel(out[0, h, t], swiglu_ref(q[0, h, t], w1[0, h], w2[0, h], w3[0, h])) < 1e-12


def _fd_total_grad(xs, vs, es, w1, w2, w3, loss, hstep=1e-6):
    """Central differences of sum_t eta_t L_t over every weight entry."""
    def total(a, b, c):
        s = 0.0
        for x, vv, e in zip(xs, vs, es):
            y = swiglu_ref(x, a, b, c)
            s += e * (0.5 * np.sum((y - vv) ** 2) if loss == 1 else -np.dot(y, vv))
        return s

    grads = []
    for which in range(3):
        W = [w1, w2, w3][which]
        G = np.zeros_like(W)
        for idx in np.ndindex(W.shape):
            ws_p = [w1.copy(), w2.copy(), w3.copy()]
            ws_m = [w1.copy(), w2.copy(), w3.copy()]
            ws_p[which][idx] += hstep
            ws_m[which][idx] -= hstep
            G[idx] = (total(*ws_p) - total(*ws_m)) / (2 * hstep)
        grads.append(G)
    return grads


@pytest.mark.parametrize("loss", [0, 1])
@pytest.mark.parametrize("rownorm", [0, 1])
def test_lact_one_update_is_gd_on_fd_gradient(loss, rownorm):
    """Section 3.2/3.3: one chunk -> W' = W - grad sum_t eta_t L_t (then row norms)."""
    rng = np.random.default_rng(32 + loss)
    T, d, hid = 3, 4, 8
    q, k, v, eta, w1, w2, w3 = rand_lact(rng, 1, 1, T, d, hid, Tq=2)
    out, f1, f2, f3 = oracle.lact_swiglu(q, k, v, eta, w1, w2, w3, chunk=T, loss=loss,
                                         order=oracle.NONCAUSAL, rownorm=rownorm)
    g1, g2, g3 = _fd_total_grad(k[0, 0], v[0, 0], eta[0, 0], w1[0, 0], w2[0, 0], w3[0, 0], loss)
    exp = []
    for W, G in ((w1[0, 0], g1), (w2[0, 0], g2), (w3[0, 0], g3)):
        Wn = W - G
        if rownorm:
            Wn = Wn * (np.linalg.norm(W, axis=1) / np.linalg.norm(Wn, axis=1))[:, None]
        exp.append(Wn)
    for got, want in zip((f1, f2, f3), exp):
        assert rel(got[0, 0], want) < 2e-7
    for t in range(2):
        assert rel(out[0, 0, t], swiglu_ref(q[0, 0, t], *exp)) < 1e-6


def test_lact_rownorm_preserves_row_norms():
    rng = np.random.default_rng(34)
    q, k, v, eta, w1, w2, w3 = rand_lact(rng, 1, 2, 20, 4, 8)
    _, f1, f2, f3 = oracle.lact_swiglu(q, k, v, eta, w1, w2, w3, chunk=6)
    for a, b in ((f1, w1), (f2, w2), (f3, w3)):
        assert rel(np.linalg.norm(a, axis=-1), np.linalg.norm(b, axis=-1)) < RTOL
    _, g1, _, _ = oracle.lact_swiglu(q, k, v, eta, w1, w2, w3, chunk=6, rownorm=0)
    assert rel(np.linalg.norm(g1, axis=-1), np.linalg.norm(w1, axis=-1)) > 1e-4


def test_lact_causal_first_chunk_and_whole_sequence_chunk():
    rng = np.random.default_rng(35)
    q, k, v, eta, w1, w2, w3 = rand_lact(rng, 1, 1, 12, 4, 8)
    out, *_ = oracle.lact_swiglu(q, k, v, eta, w1, w2, w3, chunk=5)
    for t in range(5):
        assert rel(out[0, 0, t], swiglu_ref(q[0, 0, t], w1[0, 0], w2[0, 0], w3[0, 0])) < 1e-12
    assert rel(out[0, 0, 5], swiglu_ref(q[0, 0, 5], w1[0, 0], w2[0, 0], w3[0, 0])) > 1e-6
    out_all, *_ = oracle.lact_swiglu(q, k, v, eta, w1, w2, w3, chunk=12)
    for t in range(12):
        assert rel(out_all[0, 0, t], swiglu_ref(q[0, 0, t], w1[0, 0], w2[0, 0], w3[0, 0])) < 1e-12


@pytest.mark.parametrize("loss", [0, 1])
@pytest.mark.parametrize("order", [0, 1])
def test_lact_dense_form_matches_token_loop(loss, order):
    rng = np.random.default_rng(36)
    Tq = 30 if order == 0 else 11
    q, k, v, eta, w1, w2, w3 = rand_lact(rng, 1, 2, 30, 8, 16, Tq=Tq)
    out, f1, f2, f3 = oracle.lact_swiglu(q, k, v, eta, w1, w2, w3, chunk=7, loss=loss,
                                         order=order)
    for h in range(2):
        o, a, b, c = dense.lact_head(q[0, h], k[0, h], v[0, h], eta[0, h], w1[0, h], w2[0, h],
                                     w3[0, h], chunk=7, loss=loss, order=order)
        assert rel(o, out[0, h]) < 1e-11
        assert rel(a, f1[0, h]) < 1e-11 and rel(b, f2[0, h]) < 1e-11 and rel(c, f3[0, h]) < 1e-11


def test_lact_state_carry_and_head_isolation():
    rng = np.random.default_rng(37)
    q, k, v, eta, w1, w2, w3 = rand_lact(rng, 1, 2, 24, 4, 8)
    full = oracle.lact_swiglu(q, k, v, eta, w1, w2, w3, chunk=6)
    T1 = 12
    s = lambda x, a, b: x[:, :, a:b]
    p1 = oracle.lact_swiglu(s(q, 0, T1), s(k, 0, T1), s(v, 0, T1), eta[:, :, :T1], w1, w2, w3,
                            chunk=6)
    p2 = oracle.lact_swiglu(s(q, T1, 24), s(k, T1, 24), s(v, T1, 24), eta[:, :, T1:], p1[1],
                            p1[2], p1[3], chunk=6)
    assert rel(np.concatenate([p1[0], p2[0]], axis=2), full[0]) < RTOL
    for a, b in zip(p2[1:], full[1:]):
        assert rel(a, b) < RTOL
    v2 = v.copy()
    v2[0, 1] *= 2.0
    pert = oracle.lact_swiglu(q, k, v2, eta, w1, w2, w3, chunk=6)
    assert np.array_equal(pert[0][0, 0], full[0][0, 0])
    assert not np.array_equal(pert[0][0, 1, 6:], full[0][0, 1, 6:])


def test_silu_derivative_by_finite_differences():
    """R10: silu'(z) = s (1 + z (1 - s)) -- checked through the token loop: with
    W2 = I-like single unit the gradient wrt W1 carries silu'(h1)."""
    rng = np.random.default_rng(38)
    q, k, v, eta, w1, w2, w3 = rand_lact(rng, 1, 1, 1, 1, 1)
    _, f1, _, _ = oracle.lact_swiglu(q, k, v, eta, w1, w2, w3, chunk=1, rownorm=0)
    x, vv, e = k[0, 0, 0, 0], v[0, 0, 0, 0], eta[0, 0, 0]
    a1, a2, a3 = w1[0, 0, 0, 0], w2[0, 0, 0, 0], w3[0, 0, 0, 0]
    silu = lambda z: z / (1 + np.exp(-z))
    L = lambda w: -e * a2 * silu(w * x) * (a3 * x) * vv
    hs = 1e-6
    g = (L(a1 + hs) - L(a1 - hs)) / (2 * hs)
    assert abs((f1[0, 0, 0, 0] - a1) - (-g)) < 1e-8


def test_handworked_lact_two_chunks():
    """Worked by hand (LaCT sections 3.2-3.3 and 4, readings R8 and R10):
    d = 2, hid = 1, W1 = [1, 0], W3 = [0, 1], W2 = [1, 0]^T, one key x = [1, 1],
    v = [1, 2], eta = 1/2, causal, chunk 1, rownorm on.  With s = sigmoid(1):
    h1 = h3 = 1, a = g = s, dy = -eta v = [-1/2, -1], dg = W2^T dy = -1/2,
    G2 = dy g = [-s/2, -s]^T, G3 = dg a x^T = -s/2 [1, 1],
    G1 = dg h3 silu'(1) x^T = -(s (2 - s))/2 [1, 1].
    W1' = [1 + u, u] with u = s (2 - s)/2, then scaled back to norm 1;
    W3' = [s/2, 1 + s/2] scaled back to norm 1; W2' rows: row 0 = 1 + s/2 -> |1| = 1,
    row 1 = s scaled to its old norm 0 -> 0, so W2 is unchanged.
    Outputs: y1 = f(q1; W_init) = [silu(1) * 1, 0] for q1 = [1, 1];
    y2 = f(q2; W') for q2 = [1, 1] = [silu(W1' q2) * (W3' q2), 0]."""
    import math
    s = 1.0 / (1.0 + math.exp(-1.0))
    u = s * (2.0 - s) / 2.0
    n1 = math.hypot(1.0 + u, u)
    w1n = [(1.0 + u) / n1, u / n1]
    n3 = math.hypot(s / 2.0, 1.0 + s / 2.0)
    w3n = [(s / 2.0) / n3, (1.0 + s / 2.0) / n3]
    z1 = w1n[0] + w1n[1]
    z3 = w3n[0] + w3n[1]
    silu = lambda z: z / (1.0 + math.exp(-z))
    y1 = [silu(1.0), 0.0]
    y2 = [silu(z1) * z3, 0.0]
    q = np.array([[[[1.0, 1.0], [1.0, 1.0]]]])
    k = np.array([[[[1.0, 1.0], [0.0, 0.0]]]])
    v = np.array([[[[1.0, 2.0], [0.0, 0.0]]]])
    eta = np.array([[[0.5, 0.0]]])
    w1 = np.array([[[[1.0, 0.0]]]])
    w3 = np.array([[[[0.0, 1.0]]]])
    w2 = np.array([[[[1.0], [0.0]]]])
    out, f1, f2, f3 = oracle.lact_swiglu(q, k, v, eta, w1, w2, w3, chunk=1, loss=0, order=0,
                                         rownorm=1)
    np.testing.assert_allclose(out[0, 0], [y1, y2], rtol=0, atol=1e-15)
    np.testing.assert_allclose(f1[0, 0, 0], w1n, rtol=0, atol=1e-15)
    np.testing.assert_allclose(f3[0, 0, 0], w3n, rtol=0, atol=1e-15)
    np.testing.assert_allclose(f2[0, 0, :, 0], [1.0, 0.0], rtol=0, atol=1e-15)


# --------------------------------------------------------------------------
# LaCT update rules: momentum and Muon ("LaCT" section 3.3 names gradient
# descent, momentum and Muon -- a Newton-Schulz map of the matrix gradient --
# without coefficients; the readings are beta, k steps of the cubic iteration
# from M / ||M||_F, and a step size lr).
# --------------------------------------------------------------------------
def _ns_by_svd(m, steps):
    """Closed form of k Newton-Schulz steps: X_k = U f^k(S / ||M||_F) V^T with
    f(s) = 1.5 s - 0.5 s^3, from numpy's SVD."""
    u, sv, vt = np.linalg.svd(m, full_matrices=False)
    s = sv / np.sqrt(np.sum(m * m))
    for _ in range(steps):
        s = 1.5 * s - 0.5 * s ** 3
    return (u * s) @ vt


@pytest.mark.parametrize("shape", [(12, 5), (5, 12), (9, 9)])
@pytest.mark.parametrize("steps", [1, 3, 5])
def test_newton_schulz_matches_svd_closed_form(shape, steps):
    rng = np.random.default_rng(51)
    m = rng.standard_normal(shape)
    assert rel(dense.newton_schulz(m, steps), _ns_by_svd(m, steps)) < 1e-12


def test_newton_schulz_fixed_points():
    """A rank-one matrix s u v^T maps to u v^T after any number of steps; the
    iteration converges to the polar factor; zero maps to zero."""
    rng = np.random.default_rng(52)
    u = rng.standard_normal(7)
    u /= np.linalg.norm(u)
    v = rng.standard_normal(4)
    v /= np.linalg.norm(v)
    assert rel(dense.newton_schulz(3.7 * np.outer(u, v), 5), np.outer(u, v)) < 1e-14
    m = rng.standard_normal((6, 3))
    uu, _, vt = np.linalg.svd(m, full_matrices=False)
    assert rel(dense.newton_schulz(m, 40), uu @ vt) < 1e-10
    assert np.array_equal(dense.newton_schulz(np.zeros((3, 2)), 5), np.zeros((3, 2)))


def _lact_small(seed, T=24, d=6, hid=10, B=1, H=2):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, H, T, d)) / np.sqrt(d)
    k = rng.standard_normal((B, H, T, d)) / np.sqrt(d)
    v = rng.standard_normal((B, H, T, d))
    eta = rng.uniform(0.05, 0.3, (B, H, T))
    w1 = rng.standard_normal((B, H, hid, d)) / np.sqrt(d)
    w2 = rng.standard_normal((B, H, d, hid)) / np.sqrt(hid)
    w3 = rng.standard_normal((B, H, hid, d)) / np.sqrt(d)
    return q, k, v, eta, w1, w2, w3


def _gd_gradient(k, v, eta, w1, w2, w3, loss):
    """Chunk gradients extracted from the (pinned) gradient-descent oracle: one
    chunk without the row rescale moves each W by exactly minus its gradient."""
    _, f1, f2, f3 = oracle.lact_swiglu(k[:, :, :1] * 0, k, v, eta, w1, w2, w3, chunk=k.shape[2],
                                       loss=loss, order=oracle.NONCAUSAL, rownorm=0)
    return w1 - f1, w2 - f2, w3 - f3


def test_lact_rule_gd_and_beta_zero_momentum_equal_plain_gd():
    q, k, v, eta, w1, w2, w3 = _lact_small(53)
    ref = oracle.lact_swiglu(q, k, v, eta, w1, w2, w3, chunk=8, loss=0, order=0, rownorm=1)
    for rule in (oracle.RULE_GD, oracle.RULE_MOMENTUM):
        got = oracle.lact_swiglu_rule(q, k, v, eta, w1, w2, w3, chunk=8, loss=0, order=0,
                                      rownorm=1, rule=rule, beta=0.0)
        for a, b in zip(got[:4], ref):
            assert rel(a, b) < 1e-13


@pytest.mark.parametrize("loss", [0, 1])
def test_lact_momentum_composes_gd_gradients(loss):
    """Three chunks of momentum: M_c = beta M_{c-1} + G_c(W_c), W_{c+1} = W_c - M_c,
    with every G_c taken from the gradient-descent oracle at the current weights;
    the final momentum buffers are M_2."""
    q, k, v, eta, w1, w2, w3 = _lact_small(54, T=24)
    beta, chunk = 0.6, 8
    out, f1, f2, f3, m = oracle.lact_swiglu_rule(q, k, v, eta, w1, w2, w3, chunk=chunk, loss=loss,
                                                 order=0, rownorm=0, rule=oracle.RULE_MOMENTUM,
                                                 beta=beta)
    W = [w1.copy(), w2.copy(), w3.copy()]
    M = [np.zeros_like(w1), np.zeros_like(w2), np.zeros_like(w3)]
    outs = []
    for c0 in range(0, 24, chunk):
        sl = slice(c0, c0 + chunk)
        outs.append(oracle.lact_swiglu(q[:, :, sl], k[:, :, :0], v[:, :, :0], eta[:, :, :0], *W,
                                       chunk=chunk, loss=loss, order=oracle.NONCAUSAL,
                                       rownorm=0)[0])
        G = _gd_gradient(k[:, :, sl], v[:, :, sl], eta[:, :, sl], *W, loss)
        M = [beta * a + g for a, g in zip(M, G)]
        W = [w - a for w, a in zip(W, M)]
    assert rel(out, np.concatenate(outs, axis=2)) < 1e-12
    for a, b in zip((f1, f2, f3), W):
        assert rel(a, b) < 1e-12
    for a, b in zip(m, M):
        assert rel(a, b) < 1e-12


@pytest.mark.parametrize("beta", [0.0, 0.5])
def test_lact_muon_step_is_lr_times_svd_polar_map(beta):
    """Two chunks of Muon without the row rescale: W <- W - lr * U f^k(S/||M||) V^T
    of the momentum, with gradients from the gradient-descent oracle and the
    Newton-Schulz map from numpy's SVD."""
    q, k, v, eta, w1, w2, w3 = _lact_small(55, T=16)
    lr, steps, chunk = 0.03, 5, 8
    _, f1, f2, f3, m = oracle.lact_swiglu_rule(q, k, v, eta, w1, w2, w3, chunk=chunk, loss=0,
                                               order=0, rownorm=0, rule=oracle.RULE_MUON,
                                               beta=beta, ns_steps=steps, lr=lr)
    W = [w1.copy(), w2.copy(), w3.copy()]
    M = [np.zeros_like(w1), np.zeros_like(w2), np.zeros_like(w3)]
    for c0 in range(0, 16, chunk):
        sl = slice(c0, c0 + chunk)
        G = _gd_gradient(k[:, :, sl], v[:, :, sl], eta[:, :, sl], *W, 0)
        M = [beta * a + g for a, g in zip(M, G)]
        for i in range(3):
            for h in range(2):
                W[i][0, h] = W[i][0, h] - lr * _ns_by_svd(M[i][0, h], steps)
    for a, b in zip((f1, f2, f3), W):
        assert rel(a, b) < 1e-11
    if beta:
        for a, b in zip(m, M):
            assert rel(a, b) < 1e-12


@pytest.mark.parametrize("rule,beta", [(1, 0.7), (2, 0.0), (2, 0.8)])
@pytest.mark.parametrize("order", [0, 1])
def test_lact_rule_dense_form_matches_token_loop(rule, beta, order):
    q, k, v, eta, w1, w2, w3 = _lact_small(56, T=20)
    kw = dict(chunk=8, loss=1, order=order, rownorm=1, rule=rule, beta=beta, ns_steps=3, lr=0.05)
    out, f1, f2, f3, m = oracle.lact_swiglu_rule(q, k, v, eta, w1, w2, w3, **kw)
    for h in range(2):
        mm = [np.zeros_like(w1[0, h]), np.zeros_like(w2[0, h]), np.zeros_like(w3[0, h])]
        o, a1, a2, a3 = dense.lact_head(q[0, h], k[0, h], v[0, h], eta[0, h], w1[0, h], w2[0, h],
                                        w3[0, h], m=mm, **kw)
        assert rel(o, out[0, h]) < 1e-11
        for a, b in zip((a1, a2, a3), (f1, f2, f3)):
            assert rel(a, b[0, h]) < 1e-11
        if rule == 1 or beta:
            for a, b in zip(mm, m):
                assert rel(a, b[0, h]) < 1e-11


def test_lact_momentum_state_carry():
    """Two calls carrying weights and momentum buffers = one call (chunk-aligned split)."""
    q, k, v, eta, w1, w2, w3 = _lact_small(57, T=24)
    kw = dict(chunk=8, loss=0, rownorm=1, rule=oracle.RULE_MUON, beta=0.9, ns_steps=2, lr=0.02)
    o, f1, f2, f3, m = oracle.lact_swiglu_rule(q, k, v, eta, w1, w2, w3, order=0, **kw)
    a = slice(0, 16)
    b = slice(16, 24)
    oa, g1, g2, g3, ma = oracle.lact_swiglu_rule(q[:, :, a], k[:, :, a], v[:, :, a], eta[:, :, a],
                                                 w1, w2, w3, order=0, **kw)
    ob, h1, h2, h3, mb = oracle.lact_swiglu_rule(q[:, :, b], k[:, :, b], v[:, :, b], eta[:, :, b],
                                                 g1, g2, g3, order=0, m=ma, **kw)
    assert rel(np.concatenate([oa, ob], axis=2), o) < 1e-13
    for x, y in zip((h1, h2, h3) + tuple(mb), (f1, f2, f3) + tuple(m)):
        assert rel(x, y) < 1e-13
