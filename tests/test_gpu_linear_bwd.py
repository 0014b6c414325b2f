"""GPU parity of ttt_linear_bwd against the fp64 backward oracle (same seeded
inputs and upstream gradients).

Tolerances: fp32 inputs, every gradient max |gpu - oracle| / max |oracle| <=
1e-4; bf16 inputs, d_q, d_k, d_v (rounded to bf16) within 2e-2 x RMS after
their own rounding (tests/parity.py), d_eta and d_w_init (fp32 outputs of an
fp32 computation on bf16-exact inputs) within 1e-4 normwise.
"""
import numpy as np
import pytest
import torch

import ttt_inputs as ti
from oracle.backward import ttt_linear_bwd as oracle_bwd
from tests.parity import assert_close, assert_close_bf16_rounded, dev, to_np

pytestmark = pytest.mark.gpu


def _cla():
    import chunked_linear_attention_amd as cla
    return cla


def run_case(B, H, T, chunk, loss, dtype, seed, with_dwf=True, heads=None, order=0, Tq=None,
             d=64):
    cla = _cla()
    Tq = T if Tq is None else Tq
    inp = ti.gen_linear(B, H, Tq, T, d, seed=seed, dtype=dtype, w0="normal")
    rng = np.random.default_rng(seed + 1)
    dy = rng.standard_normal((B, H, Tq, d)).astype(np.float32)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    if dtype == "bf16":
        dy = ti.round_bf16(dy)
        g_dy = dev(None, ti.f32_to_bf16_bits(dy), tdt)
    else:
        g_dy = dev(dy)
    dwf = rng.standard_normal((B, H, d, d)).astype(np.float32) if with_dwf else None
    g = {n: dev(inp[n], inp.get(n + "16"), tdt) for n in ("q", "k", "v")}
    print(f"[case] bwd B={B} H={H} T={T} Tq={Tq} b={chunk} loss={loss} {dtype} order={order} "
          f"dwf={with_dwf}", flush=True)
    out = cla.ttt_linear_bwd(g["q"], g["k"], g["v"], dev(inp["eta"]), dev(inp["w0"]), g_dy,
                             None if dwf is None else dev(dwf), chunk=chunk, loss=loss,
                             order=order)
    torch.cuda.synchronize()
    got = [to_np(t) for t in out]
    sl = slice(None) if heads is None else heads
    flat = lambda a: a.reshape((B * H,) + a.shape[2:])[sl][None]
    ref = oracle_bwd(flat(inp["q"]), flat(inp["k"]), flat(inp["v"]), flat(inp["eta"]),
                     flat(inp["w0"]), flat(dy), None if dwf is None else flat(dwf), chunk=chunk,
                     loss=loss, order=order)
    for name, a, r in zip(("d_q", "d_k", "d_v", "d_eta", "d_w_init"), got, ref):
        a = flat(a)
        if dtype == "f32" or name in ("d_eta", "d_w_init"):
            assert_close(a, r, "f32", name)
        else:
            assert_close_bf16_rounded(a, r, name)


@pytest.mark.parametrize("loss", [0, 1])
@pytest.mark.parametrize("chunk", [16, 32])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_bwd_small(loss, chunk, dtype):
    run_case(1, 2, 200, chunk, loss, dtype, seed=120 + chunk + loss)


@pytest.mark.parametrize("T", [1, 16, 50])
def test_bwd_ragged_and_tiny(T):
    run_case(2, 1, T, 32, 1, "f32", seed=130 + T, with_dwf=False)


def test_bwd_headline_shape_sampled_heads():
    """B4 H8 T4096 d64 chunk 16, MSE, bf16 (the forward's headline workload
    shape), heads 0 and 31 against the oracle."""
    run_case(4, 8, 4096, 16, 1, "bf16", seed=140, heads=[0, 31])


@pytest.mark.parametrize("loss", [0, 1])
@pytest.mark.parametrize("chunk", [16, 32])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_bwd_noncausal(loss, chunk, dtype):
    """Update over 200 key/value tokens, then 77 queries read the final state."""
    run_case(1, 2, 200, chunk, loss, dtype, seed=160 + chunk + loss, order=1, Tq=77)


def test_bwd_noncausal_many_queries_no_dwf():
    run_case(2, 1, 50, 16, 1, "f32", seed=170, with_dwf=False, order=1, Tq=300)


@pytest.mark.parametrize("loss", [0, 1])
@pytest.mark.parametrize("order", [0, 1])
def test_bwd_d128(loss, order):
    """Head dim 128 (chunk 16), both orders, ragged key/value length."""
    run_case(1, 2, 150, 16, loss, "bf16", seed=180 + loss + order, order=order,
             Tq=150 if order == 0 else 40, d=128)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_bwd_d128_f32_and_bf16_chunk16(dtype):
    """Head dim 128, chunk 16, MSE, ragged key/value length, in fp32 (held to
    1e-4 normwise) as well as bf16."""
    run_case(1, 2, 150, 16, 1, dtype, seed=185, d=128)


# Chunks of 16 k tokens beyond the whole-chunk kernels: the serial passes step
# over 16-token tiles against the chunk-start state, the G-free terms run tile
# against tile.
@pytest.mark.parametrize("loss", [0, 1])
@pytest.mark.parametrize("chunk", [48, 64, 256])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_bwd_large_chunks(loss, chunk, dtype):
    """d = 64, several chunks and a ragged tail (T = 300)."""
    run_case(1, 2, 300, chunk, loss, dtype, seed=190 + chunk + loss)


@pytest.mark.parametrize("loss", [0, 1])
@pytest.mark.parametrize("chunk", [48, 256])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_bwd_large_chunks_noncausal(loss, chunk, dtype):
    """d = 64, update-then-apply order over several chunks and a ragged tail
    (T = 300), fewer queries than keys."""
    run_case(1, 2, 300, chunk, loss, dtype, seed=260 + chunk + loss, order=1, Tq=70)


@pytest.mark.parametrize("loss", [0, 1])
@pytest.mark.parametrize("order", [0, 1])
@pytest.mark.parametrize("chunk", [32, 64, 1024])
def test_bwd_d128_large_chunks(loss, order, chunk):
    """d = 128 (chunk 32 upward runs the tiled kernels), both orders; chunk
    1024 over 1100 tokens is one whole chunk and a 76-token tail."""
    T = 1100 if chunk == 1024 else 200
    run_case(1, 2, T, chunk, loss, "bf16", seed=200 + chunk + loss + order, order=order,
             Tq=T if order == 0 else 60, d=128)


@pytest.mark.parametrize("loss", [0, 1])
@pytest.mark.parametrize("chunk", [32, 64])
def test_bwd_d128_large_chunks_f32(loss, chunk):
    """d = 128 with fp32 inputs through the tile kernels (their fp32
    instantiations hold more registers), ragged tail, held to 1e-4 normwise."""
    run_case(1, 2, 200, chunk, loss, "f32", seed=240 + chunk + loss, d=128)


@pytest.mark.parametrize("chunk", [64, 256, 1024])
def test_bwd_d128_sweep_shape_sampled_heads(chunk):
    """The chunk-size sweep's shape (B2 H16 T16384 d128, MSE, bf16) at chunks
    64, 256 and 1024; heads 0 and 31 against the oracle."""
    run_case(2, 16, 16384, chunk, 1, "bf16", seed=210 + chunk, heads=[0, 31], d=128)


# The serial recursions in segments (maps in parallel, chain, walks): shapes
# long enough for many segments per head.
@pytest.mark.parametrize("loss", [0, 1])
@pytest.mark.parametrize("chunk", [16, 32, 64])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_bwd_many_segments(loss, chunk, dtype):
    run_case(1, 2, 2000, chunk, loss, dtype, seed=220 + chunk + loss)


@pytest.mark.parametrize("loss", [0, 1])
def test_bwd_many_segments_noncausal_d128(loss):
    run_case(1, 2, 2000, 16, loss, "f32", seed=230 + loss, order=1, Tq=90, d=128)


@pytest.mark.parametrize("d,chunk,order", [(64, 16, 0), (128, 64, 0), (64, 32, 1)])
def test_bwd_repeat_runs_are_bitwise_identical(d, chunk, order):
    """Every reduction of the backward sums in a fixed order (no atomics), so
    two calls on the same inputs give the same bits."""
    cla = _cla()
    T = 600
    inp = ti.gen_linear(1, 2, T, T, d, seed=250 + d + chunk, dtype="bf16", w0="normal")
    g = {n: dev(inp[n], inp.get(n + "16"), torch.bfloat16) for n in ("q", "k", "v")}
    dy = ti.f32_to_bf16_bits(np.random.default_rng(251).standard_normal((1, 2, T, d)).astype(np.float32))
    g_dy = dev(None, dy, torch.bfloat16)
    dwf = dev(np.random.default_rng(252).standard_normal((1, 2, d, d)).astype(np.float32))
    print(f"[case] bwd repeat d={d} b={chunk} order={order}", flush=True)
    outs = [cla.ttt_linear_bwd(g["q"], g["k"], g["v"], dev(inp["eta"]), dev(inp["w0"]), g_dy, dwf,
                               chunk=chunk, loss=1, order=order) for _ in range(2)]
    torch.cuda.synchronize()
    for a, b in zip(*outs):
        assert torch.equal(a, b)
