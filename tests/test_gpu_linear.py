"""GPU parity of ttt_linear_fwd against the fp64 oracle (same seeded inputs).

Shapes span several 16-token sub-blocks, several chunks and several segments
plus ragged tails; the full-size workloads are checked on all heads (d = 64)
or on sampled heads (d = 128, every chunk size of the sweep).
"""
import numpy as np
import pytest
import torch

import oracle
import ttt_inputs as ti
from tests.parity import assert_close, inputs_to_device, to_np

pytestmark = pytest.mark.gpu


def _lib():
    import chunked_linear_attention_amd as cla
    return cla


def run_case(B, H, T, d, chunk, loss, dtype, order=0, Tq=None, seed=0, seg_tokens=None,
             eta_scale=1.0, w0="identity", qk_dist="l2", v_dist="normal", heads=None):
    cla = _lib()
    Tq = T if order == 0 else (Tq if Tq is not None else T)
    inp = ti.gen_linear(B, H, Tq, T, d, seed=seed, dtype=dtype, qk_dist=qk_dist, v_dist=v_dist,
                        w0=w0, eta_scale=eta_scale)
    g = inputs_to_device(inp, dtype)
    print(f"[case] B={B} H={H} T={T} Tq={Tq} d={d} b={chunk} loss={loss} {dtype} "
          f"order={order} seg={seg_tokens}", flush=True)
    out, wf = cla.ttt_linear_fwd(g["q"], g["k"], g["v"], g["eta"], g["w0"], chunk=chunk,
                                 loss=loss, order=order, seg_tokens=seg_tokens or 0)
    torch.cuda.synchronize()
    out, wf = to_np(out), to_np(wf)
    sl = slice(None) if heads is None else heads
    q = inp["q"].reshape(B * H, Tq, d)[sl][None]
    k = inp["k"].reshape(B * H, T, d)[sl][None]
    v = inp["v"].reshape(B * H, T, d)[sl][None]
    eta = inp["eta"].reshape(B * H, T)[sl][None]
    w0a = inp["w0"].reshape(B * H, d, d)[sl][None]
    ro, rw = oracle.ttt_linear(q, k, v, eta, w0a, chunk=chunk, loss=loss, order=order)
    go = out.reshape(B * H, Tq, d)[sl][None]
    gw = wf.reshape(B * H, d, d)[sl][None]
    assert_close(go, ro, dtype, "out")
    assert_close(gw, rw, dtype, "w_final")
    assert_close(gw - w0a, rw - w0a, dtype, "w_final - w_init")
    return go, ro


def test_tiny_dot_fp32_workload():
    """Inner-product loss, fp32, 1x1 heads, T=256, d=64, b=16 (the small workload)."""
    wl = ti.TINY_DOT
    run_case(1, 1, 256, 64, 16, 0, "f32", seed=1, qk_dist="scaled", v_dist="scaled", w0="zeros")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("loss", [0, 1])
@pytest.mark.parametrize("chunk", [16, 48])
def test_fp32_small(d, loss, chunk):
    run_case(1, 2, 203, d, chunk, loss, "f32", seed=3, seg_tokens=96 if chunk == 48 else 64)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("loss", [0, 1])
@pytest.mark.parametrize("chunk", [16, 64, 256])
def test_bf16_multi_segment(d, loss, chunk):
    run_case(2, 2, 1000, d, chunk, loss, "bf16", seed=4)


@pytest.mark.parametrize("loss", [0, 1])
@pytest.mark.parametrize("chunk", [32, 48, 64, 80, 96, 112, 160, 192])
def test_bf16_chunk_schedules(chunk, loss):
    """Chunks that put several chunks in a 64-token super-block (32), fill a
    48-token super-block (48) or a whole one (64), cut a chunk into 64-token
    pieces with a short last piece (80, 96, 112, 160, 192), across several
    segments and a ragged tail."""
    run_case(1, 3, 777, 64, chunk, loss, "bf16", seed=11)


@pytest.mark.parametrize("seg", [16, 32, 160, 4096])
def test_bf16_segment_sizes(seg):
    """Results must not depend on how the sequence is cut into segments."""
    run_case(1, 3, 700, 64, 16, 1, "bf16", seed=5, seg_tokens=seg)


@pytest.mark.parametrize("T", [1, 15, 16, 17, 33])
def test_short_and_ragged(T):
    run_case(1, 2, T, 64, 16, 1, "bf16", seed=6)
    run_case(1, 1, T, 128, 32, 0, "f32", seed=6)


@pytest.mark.parametrize("loss", [0, 1])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_noncausal(loss, dtype):
    run_case(1, 2, 500, 64, 32, loss, dtype, order=1, Tq=77, seed=7)
    run_case(1, 1, 300, 128, 16, loss, dtype, order=1, Tq=300, seed=8)


def test_noncausal_no_keys_and_causal_empty():
    cla = _lib()
    d = 64
    q = torch.randn(1, 2, 40, d, device="cuda").to(torch.bfloat16)
    e = torch.empty(1, 2, 0, d, device="cuda", dtype=torch.bfloat16)
    eta = torch.empty(1, 2, 0, device="cuda")
    w0 = torch.randn(1, 2, d, d, device="cuda")
    out, wf = cla.ttt_linear_fwd(q, e, e, eta, w0, chunk=16, loss="mse", order="noncausal")
    torch.cuda.synchronize()
    assert torch.equal(wf, w0)
    ref = (q.float().cpu().double() @ w0.cpu().double())
    assert (out.float().cpu().double() - ref).abs().max().item() <= 2e-2 * ref.pow(2).mean().sqrt().item()
    z = torch.empty(1, 2, 0, d, device="cuda", dtype=torch.bfloat16)
    out2, wf2 = cla.ttt_linear_fwd(z, z, z, eta, w0, chunk=16, loss="dot", order="causal")
    torch.cuda.synchronize()
    assert torch.equal(wf2, w0) and out2.numel() == 0


def test_in_place_state_and_resume():
    """w_final may alias w_init; two chunk-aligned calls equal one call."""
    cla = _lib()
    B, H, T, d, b = 1, 4, 640, 64, 32
    inp = ti.gen_linear(B, H, T, T, d, seed=9, dtype="bf16")
    g = inputs_to_device(inp, "bf16")
    full_o, full_w = cla.ttt_linear_fwd(g["q"], g["k"], g["v"], g["eta"], g["w0"], chunk=b, loss=1)
    w = g["w0"].clone()
    T1 = 320
    s1 = lambda x: x[:, :, :T1].contiguous()
    s2 = lambda x: x[:, :, T1:].contiguous()
    o1, _ = cla.ttt_linear_fwd(s1(g["q"]), s1(g["k"]), s1(g["v"]), s1(g["eta"]), w, chunk=b, loss=1,
                               w_final=w)
    o2, _ = cla.ttt_linear_fwd(s2(g["q"]), s2(g["k"]), s2(g["v"]), s2(g["eta"]), w, chunk=b, loss=1,
                               w_final=w)
    torch.cuda.synchronize()
    # Both runs are held to the oracle's one-call result at the parity bar (two
    # bf16-rounded GPU results may each sit up to the bar from it, on either side).
    ro, rw = oracle.ttt_linear(inp["q"], inp["k"], inp["v"], inp["eta"], inp["w0"], chunk=b, loss=1)
    for o, wf in ((full_o, full_w), (torch.cat([o1, o2], dim=2), w)):
        assert_close(to_np(o), ro, "bf16", "out")
        assert_close(to_np(wf), rw, "bf16", "w_final")


def test_repeat_runs_are_bitwise_identical():
    cla = _lib()
    inp = ti.gen_linear(2, 4, 1024, 1024, 64, seed=10, dtype="bf16")
    g = inputs_to_device(inp, "bf16")
    a = cla.ttt_linear_fwd(g["q"], g["k"], g["v"], g["eta"], g["w0"], chunk=16, loss=1)
    b = cla.ttt_linear_fwd(g["q"], g["k"], g["v"], g["eta"], g["w0"], chunk=16, loss=1)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_head_isolation_nan():
    """A NaN in one head's keys stays in that head."""
    cla = _lib()
    inp = ti.gen_linear(1, 4, 512, 512, 64, seed=11, dtype="bf16")
    g = inputs_to_device(inp, "bf16")
    g["k"][0, 2, 100, 5] = float("nan")
    out, wf = cla.ttt_linear_fwd(g["q"], g["k"], g["v"], g["eta"], g["w0"], chunk=16, loss=1)
    torch.cuda.synchronize()
    for h in (0, 1, 3):
        assert torch.isfinite(out[0, h].float()).all() and torch.isfinite(wf[0, h]).all()
    assert not torch.isfinite(wf[0, 2]).all()


def test_workload_mse_d64_full_size():
    """TTT-Linear MSE, bf16, B=4, H=8, T=4096, d=64, b=16: every head."""
    wl = ti.MSE_D64
    inp_seed = ti.WORKLOAD_SEEDS[wl.name]
    run_case(wl.B, wl.H, wl.T, wl.d, wl.chunk, wl.loss, "bf16", seed=inp_seed)


@pytest.mark.parametrize("chunk", [16, 64, 256, 1024])
def test_workload_mse_d128_full_size_sampled_heads(chunk):
    """TTT-Linear MSE, bf16, B=2, H=16, T=16384, d=128, chunk sweep: 3 heads sampled."""
    wl = ti.mse_d128(chunk)
    run_case(wl.B, wl.H, wl.T, wl.d, chunk, wl.loss, "bf16", seed=ti.WORKLOAD_SEEDS[wl.name],
             heads=[0, 13, 31])
