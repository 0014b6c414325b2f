"""GPU parity of the decode entry points (ttt_linear_decode, lact_swiglu_decode)
against the fp64 oracle on the same seeded inputs.

The decode state is fp32 and every product runs in fp32 FMA, so the state is
held to the fp32 rule (max |gpu - oracle| / max |oracle| <= 1e-4) for both
input dtypes; outputs follow the usual rule of their dtype (bf16 outputs are
rounded once from fp32).
"""
import numpy as np
import pytest
import torch

import oracle
import ttt_inputs as ti
from oracle import decode as odec
from oracle import dense
from tests.lact_rounding_model import lact_head_bf16_model
from tests.parity import assert_close, assert_lact_change, dev, to_np

pytestmark = pytest.mark.gpu


def _cla():
    import chunked_linear_attention_amd as cla
    return cla


def _tok(g, name, t):
    return g[name][:, :, t].contiguous()


def _linear_inputs(B, H, T, d, dtype, seed, w0="normal"):
    inp = ti.gen_linear(B, H, T, T, d, seed=seed, dtype=dtype, w0=w0)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    g = {n: dev(inp[n], inp.get(n + "16"), tdt) for n in ("q", "k", "v")}
    g["eta"] = dev(inp["eta"])
    g["w0"] = dev(inp["w0"])
    return inp, g


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("loss", [0, 1])
@pytest.mark.parametrize("chunk", [1, 16])
def test_linear_decode_sequence(d, dtype, loss, chunk):
    """37 tokens decoded one call at a time (ragged last chunk at chunk 16), every
    output and the final state against the oracle's decode sequence."""
    cla = _cla()
    B, H, T = 2, 3, 37
    inp, g = _linear_inputs(B, H, T, d, dtype, seed=100 + d + loss + chunk)
    print(f"[case] decode d={d} {dtype} loss={loss} chunk={chunk}", flush=True)
    w = g["w0"].clone()
    anchor = None if chunk == 1 else g["w0"].clone()
    ys = []
    for t in range(T):
        last = (t + 1) % chunk == 0 or t == T - 1
        ys.append(cla.ttt_linear_decode(_tok(g, "q", t), _tok(g, "k", t), _tok(g, "v", t),
                                        g["eta"][:, :, t].contiguous(), w, loss=loss,
                                        w_anchor=anchor, anchor_update=anchor is not None and last))
    torch.cuda.synchronize()
    y = np.stack([to_np(a) for a in ys], axis=2)
    ry, rw = odec.ttt_linear_decode_sequence(inp["q"], inp["k"], inp["v"], inp["eta"], inp["w0"],
                                             loss=loss, chunk=chunk)
    assert_close(y, ry, dtype, "decode outputs")
    assert_close(to_np(w), rw, "f32", "decode state")
    assert_close(to_np(w) - inp["w0"], rw - inp["w0"], "f32", "decode state change")
    if anchor is not None:
        assert torch.equal(anchor, w)     # the last token closed its chunk
    # the same sequence through the chunked forward of the token-loop oracle
    fy, fw = oracle.ttt_linear(inp["q"], inp["k"], inp["v"], inp["eta"], inp["w0"], chunk=chunk,
                               loss=loss)
    assert_close(y, fy, dtype, "decode outputs vs chunked oracle")


def test_linear_decode_serving_batch():
    """One MSE step of the serving-size batch (B=256, H=8, d=64, bf16), anchored,
    closing the chunk: every head against the oracle; the anchor equals the new state."""
    cla = _cla()
    B, H, d = 256, 8, 64
    inp, g = _linear_inputs(B, H, 1, d, "bf16", seed=7)
    anchor_np = (inp["w0"] + 0.01 * np.random.default_rng(8).standard_normal(inp["w0"].shape)
                 ).astype(np.float32)
    w, anchor = g["w0"].clone(), dev(anchor_np)
    print("[case] decode serving batch B=256 H=8 d=64 bf16 mse anchored", flush=True)
    y = cla.ttt_linear_decode(_tok(g, "q", 0), _tok(g, "k", 0), _tok(g, "v", 0),
                              g["eta"][:, :, 0].contiguous(), w, loss=1, w_anchor=anchor,
                              anchor_update=True)
    torch.cuda.synchronize()
    ry, rw, ra = odec.ttt_linear_decode(inp["q"][:, :, 0], inp["k"][:, :, 0], inp["v"][:, :, 0],
                                        inp["eta"][:, :, 0], inp["w0"], anchor_np, loss=1,
                                        anchor_update=True)
    assert_close(to_np(y), ry, "bf16", "outputs")
    assert_close(to_np(w), rw, "f32", "state")
    assert_close(to_np(w) - inp["w0"], rw - inp["w0"], "f32", "state change")
    assert torch.equal(anchor, w)


def test_linear_decode_anchor_handling():
    """anchor_update=0 leaves the anchor bit for bit; the inner-product loss never
    reads it (a NaN anchor changes nothing)."""
    cla = _cla()
    B, H, d = 3, 2, 128
    inp, g = _linear_inputs(B, H, 1, d, "f32", seed=9)
    args = (_tok(g, "q", 0), _tok(g, "k", 0), _tok(g, "v", 0), g["eta"][:, :, 0].contiguous())
    print("[case] decode anchor handling d=128 f32", flush=True)
    anchor = g["w0"] * 0.5
    keep = anchor.clone()
    w = g["w0"].clone()
    y = cla.ttt_linear_decode(*args, w, loss=1, w_anchor=anchor, anchor_update=False)
    torch.cuda.synchronize()
    assert torch.equal(anchor, keep)
    ry, rw, _ = odec.ttt_linear_decode(inp["q"][:, :, 0], inp["k"][:, :, 0], inp["v"][:, :, 0],
                                       inp["eta"][:, :, 0], inp["w0"], 0.5 * inp["w0"], loss=1)
    assert_close(to_np(y), ry, "f32", "outputs (anchored)")
    assert_close(to_np(w), rw, "f32", "state (anchored)")
    nan_anchor = torch.full_like(g["w0"], float("nan"))
    w2 = g["w0"].clone()
    y2 = cla.ttt_linear_decode(*args, w2, loss=0, w_anchor=nan_anchor, anchor_update=False)
    w3 = g["w0"].clone()
    y3 = cla.ttt_linear_decode(*args, w3, loss=0)
    torch.cuda.synchronize()
    assert torch.equal(y2, y3) and torch.equal(w2, w3)
    assert bool(torch.isnan(nan_anchor).all())


def _lact_weights(B, H, d, hid, seed):
    inp = ti.gen_lact(B, H, 1, 1, d, hid, seed=seed)
    return inp


@pytest.mark.parametrize("d,hid", [(64, 128), (256, 512), (384, 768), (1024, 1024)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_lact_decode_apply(d, hid, dtype):
    cla = _cla()
    B, H = 3, 2
    inp = ti.gen_lact(B, H, 1, 1, d, hid, seed=d + hid)
    q = inp["q"][:, :, 0]
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    if dtype == "bf16":
        gq = dev(None, np.ascontiguousarray(inp["q16"][:, :, 0]), tdt)
    else:
        q = q.astype(np.float32)
        gq = dev(q)
    gw = [dev(inp[n]) for n in ("w1", "w2", "w3")]
    print(f"[case] lact decode d={d} hid={hid} {dtype}", flush=True)
    y = cla.lact_swiglu_decode(gq, *gw)
    torch.cuda.synchronize()
    ref = np.zeros((B, H, d))
    for b in range(B):
        for h in range(H):
            ref[b, h] = dense.swiglu_apply(q[b, h][None].astype(np.float64), inp["w1"][b, h],
                                           inp["w2"][b, h], inp["w3"][b, h])[0]
    assert_close(to_np(y), ref, dtype, "lact decode outputs")


def test_lact_decode_sequence_matches_causal_forward():
    """Decode 320 tokens (chunks 128, 128, 64): each query through lact_swiglu_decode
    with the weights as they stand, each completed chunk through lact_swiglu_fwd
    (non-causal, no queries); all outputs and the final weights against the oracle's
    causal forward."""
    cla = _cla()
    B, H, T, d, hid, chunk = 1, 2, 320, 128, 256, 128
    inp = ti.gen_lact(B, H, T, T, d, hid, seed=31)
    bf = torch.bfloat16
    g = {n: dev(None, inp[n + "16"], bf) for n in ("q", "k", "v")}
    g["eta"] = dev(inp["eta"])
    w = [dev(inp[n]).clone() for n in ("w1", "w2", "w3")]
    print("[case] lact decode sequence T=320 d=128 hid=256", flush=True)
    ys = []
    for c0 in range(0, T, chunk):
        c1 = min(c0 + chunk, T)
        for t in range(c0, c1):
            ys.append(cla.lact_swiglu_decode(g["q"][:, :, t].contiguous(), *w))
        n = c1 - c0
        empty_q = torch.empty((B, H, 0, d), dtype=bf, device="cuda")
        _, w1n, w2n, w3n = cla.lact_swiglu_fwd(
            empty_q, g["k"][:, :, c0:c1].contiguous(), g["v"][:, :, c0:c1].contiguous(),
            g["eta"][:, :, c0:c1].contiguous(), w[0], w[1], w[2], chunk=n, loss="dot",
            order="noncausal", rownorm=True)
        w = [w1n, w2n, w3n]
    torch.cuda.synchronize()
    y = np.stack([to_np(a) for a in ys], axis=2)
    ro, r1, r2, r3 = oracle.lact_swiglu(inp["q"], inp["k"], inp["v"], inp["eta"], inp["w1"],
                                        inp["w2"], inp["w3"], chunk=chunk, loss=0, order=0,
                                        rownorm=1)
    assert_close(y, ro, "bf16", "decoded outputs")
    # the changes against the oracle's, with the bar of the bf16 rounding model
    # (the weights are updated by the same kernels as the causal forward's)
    for h in range(H):
        sub = [inp[n][0, h] for n in ("q", "k", "v", "eta", "w1", "w2", "w3")]
        model = lact_head_bf16_model(*sub, chunk=chunk, loss=0, order=0, rownorm=1)
        base = dense.swiglu_apply(sub[0].astype(np.float64), *(a.astype(np.float64) for a in sub[4:]))
        assert_lact_change(y[0, h], ro[0, h], model[0], base, f"head {h} decoded out - f(Q; W_init)",
                           output=True)
        for i, (got, ref, n) in enumerate(zip(w, (r1, r2, r3), ("w1", "w2", "w3"))):
            assert_close(to_np(got)[0, h], ref[0, h], "bf16", n)
            assert_lact_change(to_np(got)[0, h], ref[0, h], model[i + 1], sub[4 + i],
                               f"head {h} {n} - init")


def test_linear_decode_graph_replays():
    """Sixteen chunk-anchored decode steps (one 16-token chunk, closed at its last
    token) captured into a graph: every replay, from the same initial state and
    with eager work between replays, equals the eager steps bit for bit."""
    cla = _cla()
    B, H, T, d, chunk = 4, 8, 16, 64, 16
    inp, g = _linear_inputs(B, H, T, d, "bf16", seed=150)
    toks = [(_tok(g, "q", t), _tok(g, "k", t), _tok(g, "v", t), g["eta"][:, :, t].contiguous())
            for t in range(T)]
    w0 = g["w0"]
    print("[case] decode graph, 16 anchored steps, B=4 H=8 d=64 bf16", flush=True)

    def run(w, anchor, outs):
        for t in range(T):
            cla.ttt_linear_decode(*toks[t], w, loss=1, w_anchor=anchor,
                                  anchor_update=t == T - 1, out=outs[t])

    w_e, a_e = w0.clone(), w0.clone()
    outs_e = [torch.empty_like(toks[0][0]) for _ in range(T)]
    run(w_e, a_e, outs_e)
    torch.cuda.synchronize()
    w_g, a_g = w0.clone(), w0.clone()
    outs_g = [torch.empty_like(toks[0][0]) for _ in range(T)]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run(w_g, a_g, outs_g)  # warm-up before capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run(w_g, a_g, outs_g)
    for _ in range(3):
        w_g.copy_(w0)
        a_g.copy_(w0)
        for o in outs_g:
            o.fill_(0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for x, y in zip(outs_g, outs_e):
            assert torch.equal(x, y)
        assert torch.equal(w_g, w_e) and torch.equal(a_g, a_e)
        run(w0.clone(), w0.clone(), [torch.empty_like(o) for o in outs_g])  # eager work between
        torch.cuda.synchronize()
