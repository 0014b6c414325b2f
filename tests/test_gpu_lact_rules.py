"""GPU parity of lact_swiglu_fwd_rule (momentum and Muon update rules)
against the fp64 oracle on the same seeded inputs.

Tolerances are those of the gradient-descent path (tests/parity.py): outputs
and final weights within 2e-2 x RMS; the changes W_final - W_init,
O - f(Q; W_init) and M_final - M_init (momentum buffers) against the
oracle's, with the bar the bf16 rounding model sets on the same inputs.
"""
import numpy as np
import pytest
import torch

import oracle
import ttt_inputs as ti
from oracle import dense
from tests.lact_rounding_model import lact_head_bf16_model
from tests.parity import (assert_close, assert_close_floor, assert_lact_change,
                          inputs_to_device, to_np)

pytestmark = pytest.mark.gpu

RULES = {"momentum": oracle.RULE_MOMENTUM, "muon": oracle.RULE_MUON}


def _cla():
    import chunked_linear_attention_amd as cla
    return cla


def run(inp, m0, *, chunk, loss, order, rule, beta, ns_steps, lr, rownorm=1):
    cla = _cla()
    g = inputs_to_device(inp, "bf16")
    mom = None if m0 is None else [torch.from_numpy(a.astype(np.float32)).cuda() for a in m0]
    out, f1, f2, f3 = cla.lact_swiglu_fwd_rule(g["q"], g["k"], g["v"], g["eta"], g["w1"], g["w2"],
                                               g["w3"], chunk=chunk, rule=rule, beta=beta,
                                               ns_steps=ns_steps, muon_lr=lr, momentum=mom,
                                               loss=loss, order=order, rownorm=rownorm)
    torch.cuda.synchronize()
    return [to_np(t) for t in (out, f1, f2, f3)], (None if mom is None else [to_np(t) for t in mom])


def check_head(gpu, gm, ref, rm, model, mm, w0, m0, q, what=""):
    """One (batch, head).  gpu/ref/model: (out, w1, w2, w3); gm/rm/mm: the momentum
    buffers after the call (or None); w0/m0 their initial values; q the queries."""
    out, f1, f2, f3 = gpu
    ro, r1, r2, r3 = ref
    assert_close(out, ro, "bf16", what + "out")
    base = dense.swiglu_apply(np.asarray(q, np.float64), *(np.asarray(w, np.float64) for w in w0))
    assert_lact_change(out, ro, model[0], base, what + "out - f(Q; W_init)", output=True)
    for i, (n, a, b) in enumerate((("w1", f1, r1), ("w2", f2, r2), ("w3", f3, r3))):
        assert_close(a, b, "bf16", what + n)
        assert_lact_change(a, b, model[i + 1], w0[i], what + n + " - init")
    if gm is not None:
        for i, (n, a, b) in enumerate(zip(("m1", "m2", "m3"), gm, rm)):
            assert_close_floor(a, b, mm[i], what + n)
            assert_lact_change(a, b, mm[i], m0[i], what + n + " - init")


def case(rule, beta, loss, order, *, B=1, H=2, Tq=512, Tkv=512, d=128, hid=256, chunk=128,
         ns_steps=5, lr=0.02, seed=61, rownorm=1):
    print(f"[case] rule={rule} beta={beta} loss={loss} order={order} B={B} H={H} Tq={Tq} "
          f"Tkv={Tkv} d={d} hid={hid} b={chunk} ns={ns_steps} lr={lr}", flush=True)
    inp = ti.gen_lact(B, H, Tq, Tkv, d, hid, seed=seed, eta_scale=20.0)
    w0 = (inp["w1"], inp["w2"], inp["w3"])
    uses_m = rule == "momentum" or beta != 0.0
    m0 = None
    if uses_m:
        rng = np.random.default_rng(seed + 1)
        m0 = [0.01 * rng.standard_normal(w.shape) for w in w0]   # a carried-in momentum
    gpu, gm = run(inp, m0, chunk=chunk, loss=loss, order=order, rule=rule, beta=beta,
                  ns_steps=ns_steps, lr=lr, rownorm=rownorm)
    ro, r1, r2, r3, rm = oracle.lact_swiglu_rule(
        inp["q"], inp["k"], inp["v"], inp["eta"], *w0, chunk=chunk, loss=loss, order=order,
        rownorm=rownorm, rule=RULES[rule], beta=beta, ns_steps=ns_steps, lr=lr,
        m=None if m0 is None else [a.astype(np.float32) for a in m0])
    for b in range(B):
        for h in range(H):
            sub = [inp[n][b, h] for n in ("q", "k", "v", "eta", "w1", "w2", "w3")]
            mh0 = None if m0 is None else [a[b, h].astype(np.float32) for a in m0]
            mm = None if m0 is None else [a.copy() for a in mh0]
            model = lact_head_bf16_model(*sub, chunk=chunk, loss=loss, order=order,
                                         rownorm=rownorm, rule=RULES[rule], beta=beta,
                                         ns_steps=ns_steps, lr=lr, m=mm)
            check_head([a[b, h] for a in gpu], None if gm is None else [a[b, h] for a in gm],
                       [a[b, h] for a in (ro, r1, r2, r3)],
                       None if rm is None else [a[b, h] for a in rm], model, mm, sub[4:],
                       mh0, sub[0], f"[{b},{h}] ")


@pytest.mark.parametrize("loss", [0, 1])
@pytest.mark.parametrize("order", [0, 1])
def test_momentum(loss, order):
    case("momentum", 0.9, loss, order, Tq=512 if order == 0 else 200)


@pytest.mark.parametrize("beta", [0.0, 0.9])
@pytest.mark.parametrize("loss", [0, 1])
def test_muon_causal(beta, loss):
    case("muon", beta, loss, 0)


def test_muon_noncausal_ragged_no_rownorm():
    case("muon", 0.5, 0, 1, Tq=130, Tkv=600, rownorm=0, ns_steps=3, lr=0.05, seed=62)


def test_muon_wider_head_multi_tile_gram():
    """d = 256, hidden 512: 2 x 2 Gram tiles per matrix, 8 apply tiles."""
    case("muon", 0.9, 0, 0, H=1, Tq=384, Tkv=384, d=256, hid=512, seed=63)


@pytest.mark.parametrize("steps", [1, 16])
def test_muon_step_counts(steps):
    case("muon", 0.0, 0, 0, H=1, Tq=256, Tkv=256, ns_steps=steps, seed=64)


@pytest.mark.parametrize("rule,beta", [("gd", 0.0), ("momentum", 0.9), ("muon", 0.9)])
def test_state_carry_bitwise(rule, beta):
    """Two calls carrying weights and momentum buffers (chunk-aligned split) give
    bit for bit the results of one call."""
    cla = _cla()
    inp = ti.gen_lact(1, 2, 512, 512, 128, 256, seed=65, eta_scale=20.0)
    g = inputs_to_device(inp, "bf16")
    kw = dict(chunk=128, rule=rule, beta=beta, ns_steps=4, muon_lr=0.03, loss="dot",
              order="causal")
    z = lambda: [torch.zeros_like(g[n]) for n in ("w1", "w2", "w3")]
    print(f"[case] state carry, {rule} beta={beta}, 512 tokens in one call vs 256 + 256",
          flush=True)
    m_all = z()
    o_all, *w_all = cla.lact_swiglu_fwd_rule(g["q"], g["k"], g["v"], g["eta"], g["w1"], g["w2"],
                                             g["w3"], momentum=m_all, **kw)
    m = z()
    a, b = slice(0, 256), slice(256, 512)
    part = lambda n, s: g[n][:, :, s].contiguous()
    oa, *wa = cla.lact_swiglu_fwd_rule(part("q", a), part("k", a), part("v", a), part("eta", a),
                                       g["w1"], g["w2"], g["w3"], momentum=m, **kw)
    ob, *wb = cla.lact_swiglu_fwd_rule(part("q", b), part("k", b), part("v", b), part("eta", b),
                                       *wa, momentum=m, **kw)
    torch.cuda.synchronize()
    assert torch.equal(torch.cat([oa, ob], dim=2), o_all)
    for x, y in zip(list(wb) + m, list(w_all) + m_all):
        assert torch.equal(x, y)


def test_gd_rule_equals_plain_entry_point():
    cla = _cla()
    inp = ti.gen_lact(1, 2, 256, 256, 128, 256, seed=66, eta_scale=20.0)
    g = inputs_to_device(inp, "bf16")
    args = (g["q"], g["k"], g["v"], g["eta"], g["w1"], g["w2"], g["w3"])
    print("[case] rule gd vs lact_swiglu_fwd", flush=True)
    a = cla.lact_swiglu_fwd_rule(*args, chunk=128, rule="gd", beta=0.5)
    b = cla.lact_swiglu_fwd(*args, chunk=128)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_workload_lact_causal_full_size_muon():
    """The causal LM workload (H4 T32768 d256 h512 b2048) under Muon with
    momentum 0.9, 5 Newton-Schulz steps: every head against the oracle's
    chunk-matmul form; row norms of the final weights equal the initial ones."""
    wl = ti.LACT_CAUSAL
    inp = ti.gen_lact_workload(wl)
    kw = dict(rule="muon", beta=0.9, ns_steps=5, lr=0.02)
    print(f"[case] {wl.name} muon", flush=True)
    z = [np.zeros_like(inp[n]) for n in ("w1", "w2", "w3")]
    gpu, gm = run(inp, z, chunk=wl.chunk, loss=wl.loss, order=wl.order, **kw)
    out, f1, f2, f3 = gpu
    for a, w0 in ((f1, inp["w1"]), (f2, inp["w2"]), (f3, inp["w3"])):
        na, n0 = np.linalg.norm(a, axis=-1), np.linalg.norm(w0.astype(np.float64), axis=-1)
        assert np.max(np.abs(na - n0) / n0) < 1e-4
    for hh in (0, 1, 2, 3):
        print(f"[oracle] {wl.name} muon head {hh}", flush=True)
        sub = [inp[n][0, hh] for n in ("q", "k", "v", "eta", "w1", "w2", "w3")]
        kw2 = dict(chunk=wl.chunk, loss=wl.loss, order=wl.order, rownorm=wl.rownorm, rule=2,
                   beta=kw["beta"], ns_steps=kw["ns_steps"], lr=kw["lr"])
        rmh = [np.zeros_like(a, dtype=np.float64) for a in sub[4:]]
        ref = dense.lact_head(*sub, m=rmh, **kw2)
        mmh = [np.zeros(a.shape, np.float32) for a in sub[4:]]
        model = lact_head_bf16_model(*sub, m=mmh, **kw2)
        check_head((out[0, hh], f1[0, hh], f2[0, hh], f3[0, hh]), [a[0, hh] for a in gm], ref,
                   rmh, model, mmh, sub[4:], [np.zeros_like(a) for a in sub[4:]], sub[0],
                   f"head {hh} ")
