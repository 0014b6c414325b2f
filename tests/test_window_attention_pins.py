"""Pins for the sliding-window attention oracle (no GPU).

"LaCT: Test-Time Training Done Right", sections 3.1 and 4: a causal sliding
window attention over the Q, K, V the TTT layer uses.  The oracle is checked
against torch's scaled-dot-product attention on the CPU in fp64 (a library
routine: causal for a window covering the sequence, an explicit boolean band
mask otherwise), and against closed forms: a one-token window returns the
value itself, equal keys average the window's values.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle.window_attention import window_attention


def rel(a, b):
    a, b = np.asarray(a), np.asarray(b)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


def rand_qkv(seed, B=2, H=2, T=37, d=8):
    rng = np.random.default_rng(seed)
    return tuple(rng.standard_normal((B, H, T, d)) for _ in range(3))


def sdpa(q, k, v, mask=None, causal=False, scale=None):
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a))
    m = None if mask is None else torch.from_numpy(mask)
    return F.scaled_dot_product_attention(t(q), t(k), t(v), attn_mask=m, is_causal=causal,
                                          scale=scale).numpy()


@pytest.mark.parametrize("window", [37, 100])
def test_full_window_is_causal_attention(window):
    q, k, v = rand_qkv(71)
    assert rel(window_attention(q, k, v, window=window), sdpa(q, k, v, causal=True)) < 1e-12


@pytest.mark.parametrize("window", [2, 5, 16])
def test_band_mask_matches_library(window):
    q, k, v = rand_qkv(72)
    T = q.shape[2]
    t = np.arange(T)
    mask = (t[None, :] <= t[:, None]) & (t[None, :] > t[:, None] - window)
    assert rel(window_attention(q, k, v, window=window), sdpa(q, k, v, mask=mask)) < 1e-12


def test_custom_scale():
    q, k, v = rand_qkv(73)
    assert rel(window_attention(q, k, v, window=37, scale=0.3),
               sdpa(q, k, v, causal=True, scale=0.3)) < 1e-12


def test_window_one_returns_values():
    q, k, v = rand_qkv(74)
    assert rel(window_attention(q, k, v, window=1), v) < 1e-15


def test_equal_keys_average_the_window():
    q, _, v = rand_qkv(75, T=20)
    k = np.ones_like(q)
    out = window_attention(q, k, v, window=6)
    ref = np.stack([v[:, :, max(0, t - 5):t + 1].mean(axis=2) for t in range(20)], axis=2)
    assert rel(out, ref) < 1e-13


def test_sampled_rows_match_all_rows():
    q, k, v = rand_qkv(76)
    rows = [0, 5, 36]
    assert rel(window_attention(q, k, v, window=9, q_rows=rows),
               window_attention(q, k, v, window=9)[:, :, rows]) == 0.0
