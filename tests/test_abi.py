"""C ABI checks that need no GPU: the library loads, exports every function
include/ttt.h declares, and rejects bad arguments on the host with the
documented status before any HIP call (no valid device pointer is ever
passed here, and none is needed: validation fails first)."""
import ctypes
import os
import re

import pytest

from chunked_linear_attention_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x10000  # 16-byte aligned, never dereferenced: every call below fails validation


def header_functions():
    src = open(os.path.join(ROOT, "include", "ttt.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(\w+)\s*\(", src)) - {"if", "sizeof"})


def test_library_exports_every_declared_function():
    lib = _lib.load()
    names = header_functions()
    assert set(names) == set(_lib.EXPORTS), names
    for n in names:
        assert hasattr(lib, n), n
    assert lib.ttt_abi_version() == 3


def test_status_strings():
    for code in (0, -1, -2, -3, -4):
        assert _lib.status_string(code) != "unknown status"
    assert _lib.status_string(7) == "unknown status"


def lin(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, dtype=1, eta=FAKE, w_init=FAKE, out=FAKE, w_final=FAKE, B=1,
             H=1, Tq=64, Tkv=64, d=64, chunk=16, loss=1, order=0, ws=FAKE, wsb=1 << 40, stream=None)
    a.update(kw)
    return lib.ttt_linear_fwd(a["q"], a["k"], a["v"], a["dtype"], a["eta"], a["w_init"], a["out"],
                              a["w_final"], a["B"], a["H"], a["Tq"], a["Tkv"], a["d"], a["chunk"],
                              a["loss"], a["order"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), _lib.TTT_EINVAL), (dict(k=None), _lib.TTT_EINVAL), (dict(eta=None), _lib.TTT_EINVAL),
    (dict(w_init=None), _lib.TTT_EINVAL), (dict(w_final=FAKE + 4), _lib.TTT_EINVAL),
    (dict(q=FAKE + 8), _lib.TTT_EINVAL), (dict(dtype=2), _lib.TTT_EINVAL), (dict(loss=2), _lib.TTT_EINVAL),
    (dict(order=5), _lib.TTT_EINVAL), (dict(B=0), _lib.TTT_EINVAL), (dict(chunk=0), _lib.TTT_EINVAL),
    (dict(Tq=32), _lib.TTT_EINVAL), (dict(Tkv=-1, Tq=-1), _lib.TTT_EINVAL),
    (dict(d=32), _lib.TTT_EUNSUPPORTED), (dict(d=96), _lib.TTT_EUNSUPPORTED),
    (dict(chunk=8), _lib.TTT_EUNSUPPORTED), (dict(chunk=24), _lib.TTT_EUNSUPPORTED),
    # several segments, so a workspace is needed (one causal segment needs none)
    (dict(wsb=16, Tq=4096, Tkv=4096), _lib.TTT_EWORKSPACE),
    (dict(ws=None, Tq=4096, Tkv=4096), _lib.TTT_EINVAL),
])
def test_linear_validation(kw, code):
    assert lin(_lib.load(), **kw) == code


def test_linear_workspace_query():
    lib = _lib.load()
    # one head of 1024 tokens runs as several segments (a workspace is needed)
    small = lib.ttt_linear_workspace_bytes(1, 1, 1024, 1024, 64, 16, 1, 0, 1)
    big = lib.ttt_linear_workspace_bytes(4, 8, 4096, 4096, 64, 16, 1, 0, 1)
    assert 0 < small <= big
    assert lib.ttt_linear_workspace_bytes(1, 1, 256, 256, 32, 16, 1, 0, 1) == 0
    assert lib.ttt_linear_workspace_bytes(1, 1, 256, 256, 64, 16, 3, 0, 1) == 0
    # the inner-product loss needs no transition matrices
    assert lib.ttt_linear_workspace_bytes(4, 8, 4096, 4096, 64, 16, 0, 0, 1) < big


def lact(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, dtype=1, eta=FAKE, w1=FAKE, w2=FAKE, w3=FAKE, out=FAKE,
             f1=FAKE, f2=FAKE, f3=FAKE, B=1, H=1, Tq=512, Tkv=512, d=128, hid=256, chunk=128, loss=0,
             order=0, rownorm=1, ws=FAKE, wsb=1 << 40, stream=None, aux=None)
    a.update(kw)
    return lib.lact_swiglu_fwd(a["q"], a["k"], a["v"], a["dtype"], a["eta"], a["w1"], a["w2"],
                               a["w3"], a["out"], a["f1"], a["f2"], a["f3"], a["B"], a["H"],
                               a["Tq"], a["Tkv"], a["d"], a["hid"], a["chunk"], a["loss"],
                               a["order"], a["rownorm"], a["ws"], a["wsb"], a["stream"], a["aux"])


@pytest.mark.parametrize("kw,code", [
    (dict(w2=None), _lib.TTT_EINVAL), (dict(f3=FAKE + 2), _lib.TTT_EINVAL),
    (dict(rownorm=2), _lib.TTT_EINVAL), (dict(hid=0), _lib.TTT_EINVAL),
    (dict(Tq=100), _lib.TTT_EINVAL), (dict(dtype=0), _lib.TTT_EUNSUPPORTED),
    (dict(order=1, Tq=100, chunk=200), _lib.TTT_EUNSUPPORTED),
    (dict(d=64), _lib.TTT_EUNSUPPORTED), (dict(hid=2048), _lib.TTT_EUNSUPPORTED),
    (dict(chunk=64), _lib.TTT_EUNSUPPORTED), (dict(wsb=0), _lib.TTT_EWORKSPACE),
    # a second stream changes nothing about validation
    (dict(wsb=0, aux=FAKE), _lib.TTT_EWORKSPACE), (dict(w1=None, aux=FAKE), _lib.TTT_EINVAL),
])
def test_lact_validation(kw, code):
    assert lact(_lib.load(), **kw) == code


def dec(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, dtype=1, eta=FAKE, w=FAKE, anchor=None, upd=0, out=FAKE, B=1,
             H=1, d=64, loss=1, stream=None)
    a.update(kw)
    return lib.ttt_linear_decode(a["q"], a["k"], a["v"], a["dtype"], a["eta"], a["w"], a["anchor"],
                                 a["upd"], a["out"], a["B"], a["H"], a["d"], a["loss"], a["stream"])


# every case fails validation before a launch
@pytest.mark.parametrize("kw,code", [
    (dict(q=None), _lib.TTT_EINVAL), (dict(eta=None), _lib.TTT_EINVAL), (dict(w=None), _lib.TTT_EINVAL),
    (dict(out=None), _lib.TTT_EINVAL), (dict(w=FAKE + 4), _lib.TTT_EINVAL),
    (dict(dtype=3), _lib.TTT_EINVAL), (dict(loss=2), _lib.TTT_EINVAL), (dict(B=0), _lib.TTT_EINVAL),
    (dict(H=-1), _lib.TTT_EINVAL), (dict(upd=2), _lib.TTT_EINVAL), (dict(upd=1), _lib.TTT_EINVAL),
    (dict(d=32), _lib.TTT_EUNSUPPORTED), (dict(d=96), _lib.TTT_EUNSUPPORTED),
    # the anchor may not overlap the running state
    (dict(anchor=FAKE), _lib.TTT_EINVAL), (dict(anchor=FAKE + 64 * 64 * 4 - 16), _lib.TTT_EINVAL),
    (dict(anchor=FAKE + 64 * 64 * 4 + 8), _lib.TTT_EINVAL),
])
def test_linear_decode_validation(kw, code):
    assert dec(_lib.load(), **kw) == code


def lact_dec(lib, **kw):
    a = dict(q=FAKE, dtype=1, w1=FAKE, w2=FAKE, w3=FAKE, out=FAKE, B=1, H=1, d=256, hid=512, ws=FAKE,
             wsb=1 << 40, stream=None)
    a.update(kw)
    return lib.lact_swiglu_decode(a["q"], a["dtype"], a["w1"], a["w2"], a["w3"], a["out"], a["B"],
                                  a["H"], a["d"], a["hid"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), _lib.TTT_EINVAL), (dict(w2=None), _lib.TTT_EINVAL), (dict(ws=None), _lib.TTT_EINVAL),
    (dict(out=FAKE + 2), _lib.TTT_EINVAL), (dict(dtype=2), _lib.TTT_EINVAL), (dict(B=0), _lib.TTT_EINVAL),
    (dict(d=96), _lib.TTT_EUNSUPPORTED), (dict(hid=2048), _lib.TTT_EUNSUPPORTED),
    (dict(wsb=512 * 4 - 1), _lib.TTT_EWORKSPACE),
])
def test_lact_decode_validation(kw, code):
    assert lact_dec(_lib.load(), **kw) == code


def test_lact_decode_workspace_query():
    lib = _lib.load()
    assert lib.lact_swiglu_decode_workspace_bytes(64, 4, 256, 512, 1) == 64 * 4 * 512 * 4
    assert lib.lact_swiglu_decode_workspace_bytes(1, 1, 96, 512, 1) == 0
    assert lib.lact_swiglu_decode_workspace_bytes(1, 1, 256, 512, 5) == 0


def lact_rule(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, dtype=1, eta=FAKE, w1=FAKE, w2=FAKE, w3=FAKE, out=FAKE,
             f1=FAKE, f2=FAKE, f3=FAKE, B=1, H=1, Tq=512, Tkv=512, d=128, hid=256, chunk=128, loss=0,
             order=0, rownorm=1, rule=1, beta=0.9, ns=5, lr=0.02, m1=FAKE, m2=FAKE, m3=FAKE, ws=FAKE,
             wsb=0, stream=None, aux=None)
    a.update(kw)
    return lib.lact_swiglu_fwd_rule(a["q"], a["k"], a["v"], a["dtype"], a["eta"], a["w1"], a["w2"],
                                    a["w3"], a["out"], a["f1"], a["f2"], a["f3"], a["B"], a["H"],
                                    a["Tq"], a["Tkv"], a["d"], a["hid"], a["chunk"], a["loss"],
                                    a["order"], a["rownorm"], a["rule"], a["beta"], a["ns"], a["lr"],
                                    a["m1"], a["m2"], a["m3"], a["ws"], a["wsb"], a["stream"],
                                    a["aux"])


# every case fails validation before a launch (wsb = 0 ends the valid ones with EWORKSPACE)
@pytest.mark.parametrize("kw,code", [
    (dict(), _lib.TTT_EWORKSPACE),
    (dict(rule=3), _lib.TTT_EINVAL), (dict(rule=-1), _lib.TTT_EINVAL),
    (dict(beta=-0.1), _lib.TTT_EINVAL), (dict(beta=1.5), _lib.TTT_EINVAL),
    (dict(beta=float("nan")), _lib.TTT_EINVAL),
    (dict(m2=None), _lib.TTT_EINVAL), (dict(m3=FAKE + 4), _lib.TTT_EINVAL),
    (dict(rule=2, ns=0), _lib.TTT_EINVAL), (dict(rule=2, ns=17), _lib.TTT_EINVAL),
    (dict(rule=2, lr=-1.0), _lib.TTT_EINVAL), (dict(rule=2, lr=float("inf")), _lib.TTT_EINVAL),
    (dict(rule=2, lr=float("nan")), _lib.TTT_EINVAL),
    # Muon without momentum needs no buffers; gradient descent ignores beta and the buffers
    (dict(rule=2, beta=0.0, m1=None, m2=None, m3=None), _lib.TTT_EWORKSPACE),
    (dict(rule=2, beta=0.5, m1=None), _lib.TTT_EINVAL),
    (dict(rule=0, beta=7.0, m1=None, m2=None, m3=None), _lib.TTT_EWORKSPACE),
    (dict(d=64), _lib.TTT_EUNSUPPORTED),
])
def test_lact_rule_validation(kw, code):
    assert lact_rule(_lib.load(), **kw) == code


def test_lact_rule_workspace_query():
    lib = _lib.load()
    args = (1, 4, 4096, 4096, 256, 512, 2048, 0, 0, 1)
    gd = lib.lact_swiglu_rule_workspace_bytes(*args, 0)
    assert gd == lib.lact_swiglu_workspace_bytes(*args)
    assert lib.lact_swiglu_rule_workspace_bytes(*args, 1) == gd
    # Muon adds two bf16 iterate copies, the Gram matrices and their diagonal
    extra = 2 * 4 * 3 * 512 * 256 * 2 + 4 * 3 * 256 * 256 * 2 + 4 * 3 * 256 * 4
    assert extra <= lib.lact_swiglu_rule_workspace_bytes(*args, 2) - gd <= extra + 3 * 256
    assert lib.lact_swiglu_rule_workspace_bytes(*args, 3) == 0


def win(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, dtype=1, out=FAKE, B=1, H=1, T=100, d=128, window=16,
             scale=0.1, acc=0, stream=None)
    a.update(kw)
    return lib.window_attention_fwd(a["q"], a["k"], a["v"], a["dtype"], a["out"], a["B"], a["H"],
                                    a["T"], a["d"], a["window"], a["scale"], a["acc"], a["stream"])


# every case fails validation before a launch (T = 0 returns before any launch)
@pytest.mark.parametrize("kw,code", [
    (dict(q=None), _lib.TTT_EINVAL), (dict(out=FAKE + 2), _lib.TTT_EINVAL),
    (dict(dtype=4), _lib.TTT_EINVAL), (dict(B=0), _lib.TTT_EINVAL), (dict(T=-1), _lib.TTT_EINVAL),
    (dict(window=0), _lib.TTT_EINVAL), (dict(scale=0.0), _lib.TTT_EINVAL),
    (dict(scale=float("nan")), _lib.TTT_EINVAL), (dict(scale=float("inf")), _lib.TTT_EINVAL),
    (dict(acc=2), _lib.TTT_EINVAL), (dict(dtype=0), _lib.TTT_EUNSUPPORTED),
    (dict(d=96), _lib.TTT_EUNSUPPORTED), (dict(d=512), _lib.TTT_EUNSUPPORTED),
    (dict(T=0, q=None, k=None, v=None, out=None), _lib.TTT_OK),
])
def test_window_attention_validation(kw, code):
    assert win(_lib.load(), **kw) == code


def lin_bwd(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, dtype=1, eta=FAKE, w0=FAKE, do=FAKE, dwf=None, dq=FAKE, dk=FAKE,
             dv=FAKE, de=FAKE, dw0=FAKE, B=1, H=1, T=100, Tkv=None, d=64, chunk=16, loss=1, order=0,
             ws=FAKE, wsb=0, stream=None)
    a.update(kw)
    tkv = a["T"] if a["Tkv"] is None else a["Tkv"]
    return lib.ttt_linear_bwd(a["q"], a["k"], a["v"], a["dtype"], a["eta"], a["w0"], a["do"],
                              a["dwf"], a["dq"], a["dk"], a["dv"], a["de"], a["dw0"], a["B"], a["H"],
                              a["T"], tkv, a["d"], a["chunk"], a["loss"], a["order"], a["ws"],
                              a["wsb"], a["stream"])


# every case fails validation before a launch (wsb = 0 ends the valid ones with EWORKSPACE)
@pytest.mark.parametrize("kw,code", [
    (dict(), _lib.TTT_EWORKSPACE), (dict(dwf=FAKE), _lib.TTT_EWORKSPACE),
    (dict(dwf=FAKE + 4), _lib.TTT_EINVAL), (dict(do=None), _lib.TTT_EINVAL),
    (dict(de=None), _lib.TTT_EINVAL), (dict(dw0=FAKE + 8), _lib.TTT_EINVAL),
    (dict(ws=None), _lib.TTT_EINVAL), (dict(T=0), _lib.TTT_EINVAL), (dict(loss=3), _lib.TTT_EINVAL),
    (dict(dtype=5), _lib.TTT_EINVAL), (dict(d=128), _lib.TTT_EWORKSPACE),
    (dict(d=128, chunk=32), _lib.TTT_EWORKSPACE), (dict(d=96), _lib.TTT_EUNSUPPORTED),
    (dict(chunk=64), _lib.TTT_EWORKSPACE), (dict(chunk=1024), _lib.TTT_EWORKSPACE),
    (dict(chunk=8), _lib.TTT_EUNSUPPORTED), (dict(chunk=40), _lib.TTT_EUNSUPPORTED),
    (dict(order=2), _lib.TTT_EINVAL), (dict(Tkv=50), _lib.TTT_EINVAL),
    (dict(order=1, Tkv=50), _lib.TTT_EWORKSPACE), (dict(order=1, Tkv=0), _lib.TTT_EINVAL),
    (dict(order=1, T=0, Tkv=50, q=None, do=None, dq=None), _lib.TTT_EWORKSPACE),
    (dict(order=1, T=3, q=None), _lib.TTT_EINVAL),
])
def test_linear_bwd_validation(kw, code):
    assert lin_bwd(_lib.load(), **kw) == code


def _bwd_nseg(NH, nch, chunk, d):
    """Segments of the backward's serial passes: the count that minimises the
    segment's 16-token tiles x (rounds of the 2 NH (S-1) d/16 map waves +
    rounds of the NH S d/16 walk waves, 1024 at a time) + 2 (S - 1), with at
    least max(1, 64 / chunk) chunks (64 tokens) per segment."""
    slots, cols = 1024, NH * (d // 16)
    best, res = None, 1
    for s in range(1, max(1, min(64, nch // max(1, 64 // chunk))) + 1):
        sc = -(-nch // s)
        ns = -(-nch // sc)
        est = sc * (chunk // 16) * (-(-(2 * cols * (ns - 1)) // slots) + -(-(cols * ns) // slots)) + 2 * (ns - 1)
        if best is None or est < best:
            best, res = est, ns
    return res


def test_linear_bwd_workspace_query():
    lib = _lib.load()
    # per chunk and head: three fp32 d x d matrices (state, G, R) and three chunk x d ones;
    # per head: the final state and dL/dW_final, and per segment a d x 2d map and a d x d start
    def size(B, H, T, d, b):
        nch = -(-T // b)
        NH = B * H
        return NH * (nch * (3 * d * d + 3 * b * d) + 2 * d * d + _bwd_nseg(NH, nch, b, d) * 3 * d * d) * 4
    assert lib.ttt_linear_bwd_workspace_bytes(4, 8, 4096, 4096, 64, 16, 1, 0, 1) == size(4, 8, 4096, 64, 16)
    assert _bwd_nseg(32, 256, 16, 64) == 8 and _bwd_nseg(32, 1024, 16, 128) == 3
    assert _bwd_nseg(32, 16, 1024, 128) == 3 and _bwd_nseg(1, 125, 16, 64) == 9
    assert lib.ttt_linear_bwd_workspace_bytes(1, 1, 50, 50, 64, 32, 0, 0, 0) == size(1, 1, 50, 64, 32)
    assert lib.ttt_linear_bwd_workspace_bytes(1, 1, 7, 50, 64, 32, 0, 1, 0) == size(1, 1, 50, 64, 32)
    assert lib.ttt_linear_bwd_workspace_bytes(1, 1, 7, 50, 64, 32, 0, 0, 0) == 0
    assert lib.ttt_linear_bwd_workspace_bytes(1, 1, 50, 50, 64, 24, 0, 0, 0) == 0
    assert lib.ttt_linear_bwd_workspace_bytes(1, 1, 50, 50, 128, 32, 0, 0, 0) == size(1, 1, 50, 128, 32)
    assert lib.ttt_linear_bwd_workspace_bytes(2, 16, 16384, 16384, 128, 1024, 1, 0, 1) == \
        size(2, 16, 16384, 128, 1024)
    assert lib.ttt_linear_bwd_workspace_bytes(1, 1, 50, 50, 128, 16, 0, 0, 0) == size(1, 1, 50, 128, 16)
    assert lib.ttt_linear_bwd_workspace_bytes(1, 2, 2000, 2000, 64, 16, 1, 0, 0) == size(1, 2, 2000, 64, 16)


def test_linear_segment_length_argument():
    """ttt_linear_fwd_seg: a negative length is rejected before any launch; the
    workspace query follows the requested length (fewer, longer segments need
    fewer summaries), and 0 is the library's own choice."""
    lib = _lib.load()
    a = (FAKE, FAKE, FAKE, 1, FAKE, FAKE, FAKE, FAKE, 1, 1, 4096, 4096, 64, 16, 1, 0)
    assert lib.ttt_linear_fwd_seg(*a, -1, FAKE, 1 << 40, None) == _lib.TTT_EINVAL
    assert lib.ttt_linear_fwd_seg(*a, 256, FAKE, 16, None) == _lib.TTT_EWORKSPACE
    q = lambda seg: lib.ttt_linear_workspace_bytes_seg(4, 8, 4096, 4096, 64, 16, 1, 0, 1, seg)
    assert q(0) == lib.ttt_linear_workspace_bytes(4, 8, 4096, 4096, 64, 16, 1, 0, 1)
    assert q(-5) == 0
    assert q(2048) < q(256) < q(64)
    assert q(4096) == 0   # one segment per head: no summaries


def lact_bwd(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, dtype=1, eta=FAKE, w1=FAKE, w2=FAKE, w3=FAKE, do=FAKE,
             dw1=None, dw2=None, dw3=None, dq=FAKE + (1 << 24), dk=FAKE + (2 << 24),
             dv=FAKE + (3 << 24), de=FAKE + (4 << 24), g1=FAKE + (5 << 24), g2=FAKE + (6 << 24),
             g3=FAKE + (7 << 24), B=1, H=1, Tq=512, Tkv=512, d=128, hid=256, chunk=128, loss=0,
             order=0, rownorm=1, ws=FAKE, wsb=0, stream=None)
    a.update(kw)
    return lib.lact_swiglu_bwd(a["q"], a["k"], a["v"], a["dtype"], a["eta"], a["w1"], a["w2"],
                               a["w3"], a["do"], a["dw1"], a["dw2"], a["dw3"], a["dq"], a["dk"],
                               a["dv"], a["de"], a["g1"], a["g2"], a["g3"], a["B"], a["H"],
                               a["Tq"], a["Tkv"], a["d"], a["hid"], a["chunk"], a["loss"],
                               a["order"], a["rownorm"], a["ws"], a["wsb"], a["stream"])


# every case fails validation before a launch (wsb = 0 ends the valid ones with EWORKSPACE)
@pytest.mark.parametrize("kw,code", [
    (dict(), _lib.TTT_EWORKSPACE),
    (dict(dw1=FAKE), _lib.TTT_EINVAL),          # upstream weight gradients: all three or none
    (dict(dw1=FAKE, dw2=FAKE, dw3=FAKE + 4), _lib.TTT_EINVAL),
    (dict(dk=None), _lib.TTT_EINVAL), (dict(g2=FAKE + 8), _lib.TTT_EINVAL),
    (dict(loss=1), _lib.TTT_EUNSUPPORTED), (dict(dtype=0), _lib.TTT_EUNSUPPORTED),
    (dict(d=64), _lib.TTT_EUNSUPPORTED), (dict(Tq=100), _lib.TTT_EINVAL),
    (dict(Tkv=0, Tq=0), _lib.TTT_EINVAL), (dict(rownorm=3), _lib.TTT_EINVAL),
    (dict(dq=FAKE), _lib.TTT_EINVAL),           # d_q would overlap q
    (dict(order=1, Tq=0, q=None, do=None, dq=None), _lib.TTT_EWORKSPACE),
])
def test_lact_bwd_validation(kw, code):
    assert lact_bwd(_lib.load(), **kw) == code


def test_lact_bwd_workspace_query():
    lib = _lib.load()
    n = lib.lact_swiglu_bwd_workspace_bytes(1, 4, 32768, 32768, 256, 512, 2048, 0, 0, 1)
    assert n > lib.lact_swiglu_workspace_bytes(1, 4, 32768, 32768, 256, 512, 2048, 0, 0, 1)
    assert lib.lact_swiglu_bwd_workspace_bytes(1, 4, 32768, 32768, 256, 512, 2048, 1, 0, 1) == 0
