"""GPU parity of lact_swiglu_fwd against the fp64 oracle (same seeded inputs).

Small shapes go through the token-by-token C oracle; the two full-size
workloads go through the oracle's chunk-matmul form (every head; all of
their outputs and final weights).  Every case checks the outputs and final weights (2e-2 x
RMS) and the changes W_final - W_init and O - f(Q; W_init) against the
oracle's changes, with the bar the bf16 rounding model sets on the same
inputs (tests/parity.py).  Row norms of the final weights are checked against
the initial ones at full size (an invariant of the update rule).
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import dense
import ttt_inputs as ti
from tests.lact_rounding_model import lact_head_bf16_model
from tests.parity import assert_close, assert_lact_change, inputs_to_device, to_np

pytestmark = pytest.mark.gpu


def _cla():
    import chunked_linear_attention_amd as cla
    return cla


def run_gpu(inp, chunk, loss, order, rownorm):
    cla = _cla()
    g = inputs_to_device(inp, "bf16")
    out, f1, f2, f3 = cla.lact_swiglu_fwd(g["q"], g["k"], g["v"], g["eta"], g["w1"], g["w2"], g["w3"],
                                          chunk=chunk, loss=loss, order=order, rownorm=rownorm)
    torch.cuda.synchronize()
    return to_np(out), to_np(f1), to_np(f2), to_np(f3)


def check_head(gpu, ref, model, w0, q, what=""):
    """One (batch, head): gpu, ref and model are (out, w1, w2, w3); w0 the initial
    (w1, w2, w3); q that head's queries."""
    out, f1, f2, f3 = gpu
    ro, r1, r2, r3 = ref
    assert_close(out, ro, "bf16", what + "out")
    base = dense.swiglu_apply(np.asarray(q, np.float64), *(np.asarray(w, np.float64) for w in w0))
    assert_lact_change(out, ro, model[0], base, what + "out - f(Q; W_init)", output=True)
    for i, (name, a, b) in enumerate((("w1", f1, r1), ("w2", f2, r2), ("w3", f3, r3))):
        assert_close(a, b, "bf16", what + name)
        assert_lact_change(a, b, model[i + 1], w0[i], what + name + " - init")


def check(gpu, ref, inp, chunk, loss, order, rownorm):
    B, H = inp["q"].shape[:2]
    for b in range(B):
        for h in range(H):
            sub = [inp[n][b, h] for n in ("q", "k", "v", "eta", "w1", "w2", "w3")]
            model = lact_head_bf16_model(*sub, chunk=chunk, loss=loss, order=order,
                                         rownorm=rownorm)
            check_head([a[b, h] for a in gpu], [a[b, h] for a in ref], model, sub[4:], sub[0],
                       f"[{b},{h}] ")


def case(B, H, Tq, Tkv, d, hid, chunk, loss, order, rownorm=1, seed=0, eta_scale=1.0):
    print(f"[case] B={B} H={H} Tq={Tq} Tkv={Tkv} d={d} hid={hid} b={chunk} loss={loss} "
          f"order={order} rownorm={rownorm}", flush=True)
    inp = ti.gen_lact(B, H, Tq, Tkv, d, hid, seed=seed, eta_scale=eta_scale)
    gpu = run_gpu(inp, chunk, loss, order, rownorm)
    ref = oracle.lact_swiglu(inp["q"], inp["k"], inp["v"], inp["eta"], inp["w1"], inp["w2"],
                             inp["w3"], chunk=chunk, loss=loss, order=order, rownorm=rownorm)
    check(gpu, ref, inp, chunk, loss, order, rownorm)


@pytest.mark.parametrize("loss", [0, 1])
def test_causal_multi_chunk(loss):
    # eta scaled up so the updates move the weights well past bf16 noise
    case(1, 2, 512, 512, 128, 256, 128, loss, 0, seed=41, eta_scale=20.0)


def test_causal_ragged_last_chunk():
    case(1, 1, 600, 600, 128, 256, 128, 0, 0, seed=42, eta_scale=20.0)


@pytest.mark.parametrize("loss", [0, 1])
def test_noncausal_single_chunk(loss):
    case(1, 2, 77, 300, 128, 256, 4096, loss, 1, seed=43, eta_scale=20.0)


def test_noncausal_multi_chunk_no_rownorm():
    case(2, 1, 130, 384, 128, 384, 128, 0, 1, rownorm=0, seed=44, eta_scale=20.0)


def test_wider_head():
    case(1, 1, 256, 256, 256, 512, 128, 0, 0, seed=45, eta_scale=20.0)


def test_in_place_state():
    cla = _cla()
    inp = ti.gen_lact(1, 2, 384, 384, 128, 256, seed=46, eta_scale=20.0)
    g = inputs_to_device(inp, "bf16")
    ref = cla.lact_swiglu_fwd(g["q"], g["k"], g["v"], g["eta"], g["w1"], g["w2"], g["w3"], chunk=128)
    w1, w2, w3 = g["w1"].clone(), g["w2"].clone(), g["w3"].clone()
    got = cla.lact_swiglu_fwd(g["q"], g["k"], g["v"], g["eta"], w1, w2, w3, chunk=128,
                              w1_final=w1, w2_final=w2, w3_final=w3)
    torch.cuda.synchronize()
    assert torch.equal(got[0], ref[0])
    for a, b in zip((w1, w2, w3), ref[1:]):
        assert torch.equal(a, b)


def test_repeat_runs_bitwise_identical():
    cla = _cla()
    inp = ti.gen_lact(1, 2, 512, 512, 128, 256, seed=47)
    g = inputs_to_device(inp, "bf16")
    a = cla.lact_swiglu_fwd(g["q"], g["k"], g["v"], g["eta"], g["w1"], g["w2"], g["w3"], chunk=128)
    b = cla.lact_swiglu_fwd(g["q"], g["k"], g["v"], g["eta"], g["w1"], g["w2"], g["w3"], chunk=128)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def _full(wl, heads):
    inp = ti.gen_lact_workload(wl)
    gpu = run_gpu(inp, wl.chunk, wl.loss, wl.order, wl.rownorm)
    out, f1, f2, f3 = gpu
    # invariant at any size: row norms of the final weights equal the initial ones
    for a, w0 in ((f1, inp["w1"]), (f2, inp["w2"]), (f3, inp["w3"])):
        na, n0 = np.linalg.norm(a, axis=-1), np.linalg.norm(w0.astype(np.float64), axis=-1)
        assert np.max(np.abs(na - n0) / n0) < 1e-4
    B, H = wl.B, wl.H
    for hh in heads:
        b, h = divmod(hh, H)
        print(f"[oracle] {wl.name} head {hh}", flush=True)
        sub = [inp[n][b, h] for n in ("q", "k", "v", "eta", "w1", "w2", "w3")]
        kw = dict(chunk=wl.chunk, loss=wl.loss, order=wl.order, rownorm=wl.rownorm)
        ref = dense.lact_head(*sub, **kw)
        model = lact_head_bf16_model(*sub, **kw)
        check_head((out[b, h], f1[b, h], f2[b, h], f3[b, h]), ref, model, sub[4:], sub[0],
                   f"head {hh} ")


def test_workload_lact_causal_full_size():
    """LaCT causal, d=256, hidden 512, b=2048, 4 heads, T=32768 (every head)."""
    _full(ti.LACT_CAUSAL, [0, 1, 2, 3])


def test_workload_lact_noncausal_full_size():
    """LaCT non-causal, d=384, hidden 768, 65536 update tokens, 16384 queries (both heads)."""
    _full(ti.LACT_NONCAUSAL, [0, 1])


def _causal_dot_inputs(seed):
    inp = ti.gen_lact(1, 2, 512, 512, 128, 256, seed=seed, eta_scale=20.0)
    return inputs_to_device(inp, "bf16")


def _call(g, aux="auto"):
    cla = _cla()
    return cla.lact_swiglu_fwd(g["q"], g["k"], g["v"], g["eta"], g["w1"], g["w2"], g["w3"],
                               chunk=128, loss=0, order=0, rownorm=1, aux_stream=aux)


def test_causal_second_stream_matches_single_stream():
    """The applies on a second stream (the binding's, or one of the caller's)
    give bit for bit the results of the single-stream schedule."""
    g = _causal_dot_inputs(64)
    one = [to_np(x) for x in _call(g, aux=None)]
    own = torch.cuda.Stream()
    torch.cuda.synchronize()
    for aux in ("auto", own):
        got = [to_np(x) for x in _call(g, aux=aux)]
        torch.cuda.synchronize()
        for x, y in zip(got, one):
            assert np.array_equal(x, y)


def test_causal_concurrent_streams():
    """Two causal inner-product calls on two streams at once (their chunk
    applies share the binding's second stream) give the results of the same
    calls made one at a time."""
    ga, gb = _causal_dot_inputs(61), _causal_dot_inputs(62)
    ref_a = [to_np(x) for x in _call(ga)]
    ref_b = [to_np(x) for x in _call(gb)]
    torch.cuda.synchronize()
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(sa):
        ra = _call(ga)
    with torch.cuda.stream(sb):
        rb = _call(gb)
    torch.cuda.synchronize()
    for x, y in zip(ra, ref_a):
        assert np.array_equal(to_np(x), y)
    for x, y in zip(rb, ref_b):
        assert np.array_equal(to_np(x), y)


def test_causal_graph_replays():
    """A causal inner-product call captured into a graph (every launch on the
    capturing stream) matches the eager call on every replay, with eager work
    and synchronisations between the replays."""
    g = _causal_dot_inputs(63)
    ref = [to_np(x) for x in _call(g)]
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        _call(g)  # warm-up on the side stream, as torch advises before capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        outs = _call(g)
    for _ in range(3):
        for t in outs:
            t.fill_(0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for x, y in zip(outs, ref):
            assert np.array_equal(to_np(x), y)
        _call(g)  # eager work between replays
        torch.cuda.synchronize()
