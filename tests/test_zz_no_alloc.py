"""ttt_linear_fwd_noalloc (the entry point for callers that cannot allocate)
against ttt_linear_fwd, through the C ABI: the same kernels, with the state
scan's scratch in the library's static device array instead of a workspace.
Two calls in a row, the second on a smaller input (the array keeps the first
call's contents, which the second must not depend on); each result must equal
the workspace entry point's bit for bit and the oracle's to the bf16 bar."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import ttt_inputs as ti
from tests.parity import assert_close, inputs_to_device, to_np

pytestmark = pytest.mark.gpu


def _noalloc(lib, g, B, H, T, d, chunk, loss, order=0):
    out = torch.empty_like(g["q"])
    wf = torch.empty_like(g["w0"])
    st = torch.cuda.current_stream().cuda_stream
    rc = lib.ttt_linear_fwd_noalloc(g["q"].data_ptr(), g["k"].data_ptr(), g["v"].data_ptr(), 1,
                                    g["eta"].data_ptr(), g["w0"].data_ptr(), out.data_ptr(),
                                    wf.data_ptr(), B, H, T, T, d, chunk, loss, order, st)
    return rc, out, wf


@pytest.mark.parametrize("loss", [1, 0])
def test_noalloc_matches_workspace_entry_point(loss):
    import chunked_linear_attention_amd as cla
    from chunked_linear_attention_amd import _lib
    lib = _lib.load()
    assert lib.ttt_linear_noalloc_max_scratch_bytes() == 64 << 20
    # first the headline shape (several segments per head: the scratch holds
    # the segment summaries), then a smaller, ragged one with fewer heads
    for (B, H, T, d, chunk, seed) in ((4, 8, 4096, 64, 16, 71), (1, 3, 1000, 64, 32, 72)):
        print(f"[case] noalloc B={B} H={H} T={T} d={d} b={chunk} loss={loss}", flush=True)
        inp = ti.gen_linear(B, H, T, T, d, seed=seed, dtype="bf16")
        g = inputs_to_device(inp, "bf16")
        rc, out, wf = _noalloc(lib, g, B, H, T, d, chunk, loss)
        assert rc == 0, _lib.status_string(rc)
        ref_o, ref_w = cla.ttt_linear_fwd(g["q"], g["k"], g["v"], g["eta"], g["w0"], chunk=chunk,
                                          loss=loss)
        torch.cuda.synchronize()
        assert torch.equal(out, ref_o) and torch.equal(wf, ref_w)
        # and the oracle on sampled heads, to the bf16 bar
        heads = [0, B * H - 1]
        sl = lambda a, n: a.reshape((B * H,) + a.shape[2:])[heads][None]
        ro, rw = oracle.ttt_linear(sl(inp["q"], 0), sl(inp["k"], 0), sl(inp["v"], 0),
                                   sl(inp["eta"], 0), sl(inp["w0"], 0), chunk=chunk, loss=loss)
        go = to_np(out).reshape((B * H, T, d))[heads][None]
        gw = to_np(wf).reshape((B * H, d, d))[heads][None]
        assert_close(go, ro, "bf16", "noalloc out")
        assert_close(gw, rw, "bf16", "noalloc w_final")


def test_noalloc_rejects_beyond_scratch():
    """An update-then-apply call summarises every head's segment, so 1024 heads
    at d = 128 need about 100 MB of scratch: more than the array holds.  The
    call must refuse (TTT_EWORKSPACE) before anything is launched; the pointers
    are placeholders that are never dereferenced."""
    from chunked_linear_attention_amd import _lib
    lib = _lib.load()
    need = lib.ttt_linear_workspace_bytes(1, 1024, 256, 256, 128, 16, 1, 1, 1)
    assert need > lib.ttt_linear_noalloc_max_scratch_bytes()
    fake = 0x10000
    rc = lib.ttt_linear_fwd_noalloc(fake, fake, fake, 1, fake, fake, fake, fake, 1, 1024, 256, 256,
                                    128, 16, 1, 1, None)
    assert rc == _lib.TTT_EWORKSPACE
