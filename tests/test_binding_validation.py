"""The Python binding checks every tensor's shape and dtype before it hands a
pointer to the library (the C ABI sees only pointers and sizes, so a tensor of
the wrong size would be read or written out of bounds on the GPU).  These
checks run before the device check, so they are exercised here with CPU
tensors: each call must raise ValueError naming the offending tensor, and no
kernel is ever reached."""
import pytest
import torch

import chunked_linear_attention_amd as cla

bf, f32 = torch.bfloat16, torch.float32


def z(*shape, dtype=f32):
    return torch.zeros(shape, dtype=dtype)


def lin_args(B=1, H=2, T=32, d=64):
    return dict(q=z(B, H, T, d, dtype=bf), k=z(B, H, T, d, dtype=bf), v=z(B, H, T, d, dtype=bf),
                eta=z(B, H, T), w_init=z(B, H, d, d))


@pytest.mark.parametrize("name,bad", [
    ("k", z(1, 2, 32, 32, dtype=bf)), ("v", z(1, 1, 32, 64, dtype=bf)),
    ("eta", z(1, 2, 31)), ("w_init", z(2, 64, 64)), ("w_init", z(1, 2, 64, 64, dtype=bf)),
    ("v", z(1, 2, 32, 64)), ("out", z(1, 2, 32, 64)), ("w_final", z(1, 2, 64, 32)),
])
def test_ttt_linear_fwd_rejects(name, bad):
    a = lin_args()
    if name in ("out", "w_final"):
        kw = {name: bad}
    else:
        a[name] = bad
        kw = {}
    with pytest.raises(ValueError, match=name):
        cla.ttt_linear_fwd(a["q"], a["k"], a["v"], a["eta"], a["w_init"], chunk=16, **kw)


def lact_args(B=1, H=1, T=128, d=128, hid=256):
    return dict(q=z(B, H, T, d, dtype=bf), k=z(B, H, T, d, dtype=bf), v=z(B, H, T, d, dtype=bf),
                eta=z(B, H, T), w1=z(B, H, hid, d), w2=z(B, H, d, hid), w3=z(B, H, hid, d))


@pytest.mark.parametrize("name,bad", [
    ("w2", z(1, 1, 256, 128)), ("w3", z(1, 1, 128, 128)), ("eta", z(1, 1, 64)),
    ("k", z(1, 1, 128, 256, dtype=bf)), ("w1", z(1, 1, 256, 128, dtype=bf)),
])
@pytest.mark.parametrize("rule", [False, True])
def test_lact_rejects_inputs(name, bad, rule):
    a = lact_args()
    a[name] = bad
    fn = cla.lact_swiglu_fwd_rule if rule else cla.lact_swiglu_fwd
    with pytest.raises(ValueError, match=name):
        fn(a["q"], a["k"], a["v"], a["eta"], a["w1"], a["w2"], a["w3"], chunk=128)


@pytest.mark.parametrize("name,bad", [
    ("out", z(1, 1, 128, 128)), ("w1_final", z(1, 1, 128, 256)), ("w2_final", z(1, 1, 256, 256)),
])
def test_lact_rejects_outputs(name, bad):
    a = lact_args()
    with pytest.raises(ValueError, match=name):
        cla.lact_swiglu_fwd(a["q"], a["k"], a["v"], a["eta"], a["w1"], a["w2"], a["w3"],
                            chunk=128, **{name: bad})


def test_lact_rule_rejects_momentum_shape():
    a = lact_args()
    mom = (z(1, 1, 256, 128), z(1, 1, 256, 128), z(1, 1, 256, 128))  # m2 must be [d][hid]
    with pytest.raises(ValueError, match="m2"):
        cla.lact_swiglu_fwd_rule(a["q"], a["k"], a["v"], a["eta"], a["w1"], a["w2"], a["w3"],
                                 chunk=128, rule="momentum", beta=0.9, momentum=mom)


def test_decode_rejects():
    q = z(2, 3, 64, dtype=bf)
    with pytest.raises(ValueError, match="w"):
        cla.ttt_linear_decode(q, q, q, z(2, 3), z(2, 3, 64, 32))
    with pytest.raises(ValueError, match="eta"):
        cla.ttt_linear_decode(q, q, q, z(3, 2), z(2, 3, 64, 64))
    with pytest.raises(ValueError, match="w2"):
        cla.lact_swiglu_decode(z(1, 1, 128, dtype=bf), z(1, 1, 256, 128), z(1, 1, 256, 128),
                               z(1, 1, 256, 128))


def test_bwd_and_window_reject():
    a = lin_args()
    with pytest.raises(ValueError, match="d_out"):
        cla.ttt_linear_bwd(a["q"], a["k"], a["v"], a["eta"], a["w_init"], z(1, 2, 16, 64, dtype=bf),
                           chunk=16)
    with pytest.raises(ValueError, match="d_w_final"):
        cla.ttt_linear_bwd(a["q"], a["k"], a["v"], a["eta"], a["w_init"], a["q"],
                           z(1, 2, 64, 64, dtype=bf), chunk=16)
    with pytest.raises(ValueError, match="k"):
        cla.window_attention_fwd(a["q"], z(1, 2, 16, 64, dtype=bf), a["v"], window=8)
