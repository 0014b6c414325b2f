"""GPU parity of window_attention_fwd against the fp64 oracle (same seeded
inputs; bf16 rule after the output's own rounding: every element within
2^-8 |oracle| + 2e-2 x RMS(oracle), see tests/parity.py).

Shapes span several 128-query workgroups and 64-key blocks with ragged ends,
windows from one token to more than the sequence, every supported head
dimension, the accumulate mode on top of a LaCT output, and the LaCT LM
workload's shape (H4 T32768 d256, window 2048) on sampled queries.
"""
import numpy as np
import pytest
import torch

import ttt_inputs as ti
from oracle.window_attention import window_attention
from tests.parity import assert_close_bf16_rounded, dev, to_np

pytestmark = pytest.mark.gpu


def _cla():
    import chunked_linear_attention_amd as cla
    return cla


def _inputs(B, H, T, d, seed):
    inp = ti.gen_lact(B, H, T, T, d, 128, seed=seed)
    g = {n: dev(None, inp[n + "16"], torch.bfloat16) for n in ("q", "k", "v")}
    return inp, g


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("T,window", [(1, 1), (37, 5), (200, 64), (300, 100), (300, 1),
                                      (260, 1000)])
def test_window_attention(d, T, window):
    cla = _cla()
    inp, g = _inputs(1, 2, T, d, seed=80 + T + window)
    # L2-normalised q and k give soft scores; a larger scale sharpens them
    scale = 4.0
    print(f"[case] window attention d={d} T={T} W={window}", flush=True)
    out = cla.window_attention_fwd(g["q"], g["k"], g["v"], window=window, scale=scale)
    torch.cuda.synchronize()
    ref = window_attention(inp["q"], inp["k"], inp["v"], window=window, scale=scale)
    assert_close_bf16_rounded(to_np(out), ref, f"window attention d={d} T={T} W={window}")


def test_window_attention_accumulates_onto_lact_output():
    """out = LaCT causal output + window attention on the same Q, K, V."""
    cla = _cla()
    B, H, T, d, hid, chunk, W = 1, 2, 384, 128, 256, 128, 128
    inp = ti.gen_lact(B, H, T, T, d, hid, seed=90, eta_scale=20.0)
    g = {n: dev(None, inp[n + "16"], torch.bfloat16) for n in ("q", "k", "v")}
    for n in ("eta", "w1", "w2", "w3"):
        g[n] = dev(inp[n])
    print("[case] LaCT causal + window attention (accumulate)", flush=True)
    out, *_ = cla.lact_swiglu_fwd(g["q"], g["k"], g["v"], g["eta"], g["w1"], g["w2"], g["w3"],
                                  chunk=chunk)
    lact_only = out.clone()
    cla.window_attention_fwd(g["q"], g["k"], g["v"], window=W, out=out, accumulate=True)
    torch.cuda.synchronize()
    ref = window_attention(inp["q"], inp["k"], inp["v"], window=W) + to_np(lact_only)
    assert_close_bf16_rounded(to_np(out), ref, "LaCT + window attention")


def test_window_attention_workload_shape_sampled():
    """H4 T32768 d256, window 2048 (the LaCT LM layer's shape): 96 sampled queries
    (sequence start, window edges, workgroup and block boundaries, the end)."""
    cla = _cla()
    B, H, T, d, W = 1, 4, 32768, 256, 2048
    inp, g = _inputs(B, H, T, d, seed=91)
    print("[case] window attention H4 T32768 d256 W2048", flush=True)
    out = to_np(cla.window_attention_fwd(g["q"], g["k"], g["v"], window=W))
    torch.cuda.synchronize()
    rng = np.random.default_rng(92)
    rows = sorted(set([0, 1, 63, 64, 127, 128, 2047, 2048, 2049, 4095, 16383, 32767] +
                      rng.integers(0, T, 84).tolist()))
    ref = window_attention(inp["q"], inp["k"], inp["v"], window=W, q_rows=rows)
    assert_close_bf16_rounded(out[:, :, rows], ref, "sampled rows")


def test_window_attention_full_window_repeatable():
    cla = _cla()
    inp, g = _inputs(2, 1, 500, 128, seed=93)
    print("[case] repeat bitwise", flush=True)
    a = cla.window_attention_fwd(g["q"], g["k"], g["v"], window=500)
    b = cla.window_attention_fwd(g["q"], g["k"], g["v"], window=10**6)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
