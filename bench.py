"""Benchmark of the TTT-layer forward on one MI355X.

Default workload: TTT-Linear, MSE loss, bf16 inputs with fp32 state, B=4,
H=8, T=4096, d=64, chunk 16 (causal).  One step = one ttt_linear_fwd call
over the whole batch (all of the path's kernels), inputs already in HBM.

Prints ONE JSON line: tokens/s (B*T per step), ms per step, the roofline of
the call (algorithmic HBM bytes per call / average call time, measured with
HIP events on the stream the library launches on), the chunk-size curve of
the d=128 workload, the LaCT workloads, and the CPU oracle timed on a bounded
sample on the host.

Algorithmic bytes of one TTT-Linear call: every head-token reads q, k, v and
eta and writes o once; every head reads the initial state and writes the final
state once:  NH*T*((3 + 1)*d*s_in + 4) + NH*2*d*d*4.
Input sets are rotated (>= 1 GiB in total) so the 256 MiB last-level cache
cannot hold the working set across steps.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0      # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published
FP32_PEAK_TFLOPS = 157.3   # MI355X fp32 matrix, published
METRIC = "TTT-layer fwd tokens/s + % of roofline (HBM or MFMA) vs chunk size, 1 GPU"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def linear_alg_bytes(NH, Tq, Tkv, d, esz):
    return NH * Tkv * (2 * d * esz + 4) + NH * Tq * 2 * d * esz + NH * 2 * d * d * 4


def linear_alg_flops(NH, T, d, b, loss):
    """Dual-form count: per chunk 2*b*d^2*(3 MSE | 2 DOT) + 2*d*b(b+1)."""
    full, rem = divmod(T, b)
    f = 0
    for n, cnt in ((b, full), (rem, 1 if rem else 0)):
        f += cnt * (2 * n * d * d * (3 if loss == 1 else 2) + 2 * d * n * (n + 1))
    return NH * f


def kernel_source_hash(names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "chunked_linear_attention_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic(kind: str, workload: str, src_hash: str):
    """HBM bytes per call from a committed rocprofv3 --pmc summary, if it was taken on
    the current kernel sources (else None)."""
    path = os.path.join(ROOT, "profiles", f"{workload}_traffic.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    if vals.get("kernel_source_sha256_16") != src_hash:
        return None
    try:
        return float(vals["hbm_bytes_per_call"])
    except (KeyError, ValueError):
        return None


class Rotated:
    """R copies of a workload's device inputs/outputs, cycled step by step."""

    def __init__(self, make_copy, bytes_per_copy, min_total=1 << 30, max_copies=16):
        import math
        self.n = max(1, min(max_copies, math.ceil(min_total / max(bytes_per_copy, 1))))
        self.sets = [make_copy(i) for i in range(self.n)]

    def __getitem__(self, i):
        return self.sets[i % self.n]


SPIN_UP_S = 0.2


def spin_up(seconds=SPIN_UP_S):
    """Keep the matrix cores busy for about `seconds` (back-to-back launches of
    the library's MFMA loop, ttt_probe_mfma_bf16) so that the timed calls do
    not start from the clocks of an idle GPU: measured after a second of idle,
    the first ~50 ms of TTT-Linear calls run up to 25% slower than the rate the
    part settles at.  No part of any timed workload runs here."""
    import torch
    import chunked_linear_attention_amd._lib as L
    lib = L.load()
    st = torch.cuda.current_stream()
    out = torch.empty(2048 * 256, device="cuda")
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(8):
            if lib.ttt_probe_mfma_bf16(out.data_ptr(), 2048, 2000, st.cuda_stream) != 0:
                raise RuntimeError("ttt_probe_mfma_bf16 failed")
        torch.cuda.synchronize()


def time_calls(fn, sets, steps, warmup):
    """Spin the GPU up (spin_up), warm up, then time exactly `steps` calls between two device syncs with
    HIP events recorded on the current stream (the one the library launches
    on), only before the first and after the last call, so nothing but the
    calls runs in between.  A second pass of the same calls records an event
    between consecutive calls for each call's own duration (the median).
    Returns (mean ms per call over the bracketed region of the first pass,
    median ms per call of the second, wall seconds of the first pass's timed
    region)."""
    import torch
    spin_up()
    for i in range(warmup):
        fn(sets[i])
    torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(st)
    for i in range(steps):
        fn(sets[i])
    e1.record(st)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    mean = e0.elapsed_time(e1) / steps
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    ev[0].record(st)
    for i in range(steps):
        fn(sets[i])
        ev[i + 1].record(st)
    torch.cuda.synchronize()
    per = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(steps))
    mid = steps // 2
    median = per[mid] if steps % 2 else 0.5 * (per[mid - 1] + per[mid])
    return mean, median, wall


# The pages' benchmark method: 10 warm-up calls, then 100 timed calls with the
# device synchronised on both sides.  Every workload besides the headline (whose
# step count the caller sets) is timed that way.
EXTRA_WARMUP, EXTRA_STEPS = 10, 100


def measured_peaks():
    """Peaks measured in this process: HBM bandwidth of a plain 1 GiB device copy
    (torch's copy kernel; bytes read + written over the copy's time, best of 5)
    and the dense bf16 rate of an MFMA loop (ttt_probe_mfma_bf16: 2048
    workgroups of four waves, four independent 32x32x16 products per wave and
    round, best of 5)."""
    import torch
    import chunked_linear_attention_amd._lib as L
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    st = torch.cuda.current_stream()
    best = None
    for _ in range(6):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(st)
        dst.copy_(src)
        e1.record(st)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
        best = ms if best is None else min(best, ms)
    copy_gbs = 2 * n / (best * 1e-3) / 1e9
    del src, dst
    blocks, iters = 2048, 2048
    out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    lib = L.load()
    best = None
    for _ in range(6):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(st)
        rc = lib.ttt_probe_mfma_bf16(out.data_ptr(), blocks, iters, st.cuda_stream)
        e1.record(st)
        torch.cuda.synchronize()
        if rc != 0:
            raise RuntimeError(f"ttt_probe_mfma_bf16 failed ({rc})")
        ms = e0.elapsed_time(e1)
        best = ms if best is None else min(best, ms)
    mfma_tflops = blocks * 4 * iters * 4 * 32768 / (best * 1e-3) / 1e12
    return {"hbm_copy_gbs": copy_gbs, "bf16_mfma_tflops": mfma_tflops,
            "method": "best of 6: 1 GiB device copy (read + write bytes); bf16 32x32x16 MFMA loop, "
                      "2048 workgroups x 4 waves x 2048 rounds x 4 products"}


def gemm_probe(steps=20, warmup=3):
    """The LaCT kernels' shared GEMM tile (128 x 128 blocks of four or eight
    waves, 256 x 128 and 64 x 128 blocks of four) on plain bf16 products
    (ttt_probe_gemm_bf16, fp32 out), beside the vendor GEMM
    behind torch.matmul on the same shapes (bf16 in and out) for context; each
    checked against an fp32 product of the same bf16 values on a small shape
    first."""
    import torch
    import chunked_linear_attention_amd._lib as L
    lib = L.load()
    st = torch.cuda.current_stream()

    def ours(a, b, c, M, N, K, ak, bk, rows=128, groups=1):
        rc = lib.ttt_probe_gemm_bf16(a.data_ptr(), b.data_ptr(), c.data_ptr(), M, N, K, ak, bk, rows, groups,
                                     st.cuda_stream)
        if rc != 0:
            raise RuntimeError(f"ttt_probe_gemm_bf16 failed ({rc})")

    def timed(fn):
        for _ in range(warmup):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(st)
        for _ in range(steps):
            fn()
        e1.record(st)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    g = torch.Generator(device="cuda").manual_seed(5)
    out = []
    for (M, N, K, ak, bk) in [(512, 384, 320, 0, 0), (512, 384, 320, 1, 1), (512, 384, 320, 0, 1)]:
        a = torch.randn((K, M) if ak else (M, K), device="cuda", generator=g).to(torch.bfloat16)
        b = torch.randn((K, N) if bk else (N, K), device="cuda", generator=g).to(torch.bfloat16)
        ref = (a.float().t() if ak else a.float()) @ (b.float() if bk else b.float().t())
        for rows, groups in ((128, 1), (256, 1), (64, 1), (128, 2)):
            c = torch.empty(M, N, device="cuda")
            ours(a, b, c, M, N, K, ak, bk, rows, groups)
            torch.cuda.synchronize()
            err = float((c - ref).abs().max() / ref.abs().max())
            if err > 1e-5:
                raise RuntimeError(f"GEMM tile probe mismatch {err:.2e} at {M}x{N}x{K} ({ak}, {bk}), "
                                   f"{rows}-row blocks, {groups} wave groups")
    for (M, N, K, ak, bk, what) in [(4096, 4096, 4096, 0, 0, "square, both operands k-contiguous"),
                                    (4096, 4096, 4096, 1, 1, "square, both operands k-major"),
                                    (8192, 8192, 8192, 0, 0, "square 8192, k-contiguous"),
                                    (16384, 1024, 256, 0, 0, "LaCT key-forward aspect (tokens x hidden x d)"),
                                    (1024, 512, 32768, 0, 1, "LaCT weight-gradient aspect (hidden x d x tokens)"),
                                    (2048, 2048, 768, 0, 1, "one tile per CU, 768-deep (LaCT backward GEMMs)"),
                                    (768, 1024, 512, 1, 1, "48 tiles, 512-deep (Newton-Schulz Gram)")]:
        a = torch.randn((K, M) if ak else (M, K), device="cuda", generator=g).to(torch.bfloat16)
        b = torch.randn((K, N) if bk else (N, K), device="cuda", generator=g).to(torch.bfloat16)
        c = torch.empty(M, N, device="cuda")
        ms = timed(lambda: ours(a, b, c, M, N, K, ak, bk))
        ms_w = timed(lambda: ours(a, b, c, M, N, K, ak, bk, 256)) if M % 256 == 0 else float("nan")
        ms_2 = timed(lambda: ours(a, b, c, M, N, K, ak, bk, 128, 2))
        ms_n = timed(lambda: ours(a, b, c, M, N, K, ak, bk, 64))
        at = a.t() if ak else a
        bt = b if bk else b.t()
        at, bt = at.contiguous(), bt.contiguous()
        vms = timed(lambda: torch.matmul(at, bt))
        fl = 2.0 * M * N * K
        out.append({"shape": f"{M}x{N}x{K}", "layout": what, "tile_us": ms * 1e3,
                    "tile_tflops": fl / (ms * 1e-3) / 1e12, "tile_frac": fl / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
                    "wide_tile_us": ms_w * 1e3, "wide_tile_tflops": fl / (ms_w * 1e-3) / 1e12,
                    "eight_wave_tile_us": ms_2 * 1e3, "eight_wave_tile_tflops": fl / (ms_2 * 1e-3) / 1e12,
                    "narrow_tile_us": ms_n * 1e3, "narrow_tile_tflops": fl / (ms_n * 1e-3) / 1e12,
                    "vendor_us": vms * 1e3, "vendor_tflops": fl / (vms * 1e-3) / 1e12})
        del a, b, c, at, bt
    return out


# ----------------------------------------------------------------------------
def linear_sets(inp, dtype, R_min_bytes):
    import numpy as np
    import torch
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32

    def up(name):
        if dtype == "bf16":
            return torch.from_numpy(inp[name + "16"].view(np.int16).copy()).view(torch.bfloat16).cuda()
        return torch.from_numpy(inp[name]).cuda()

    base = {n: up(n) for n in ("q", "k", "v")}
    base["eta"] = torch.from_numpy(inp["eta"]).cuda()
    base["w0"] = torch.from_numpy(inp["w0"]).cuda()
    per = sum(t.numel() * t.element_size() for t in base.values()) + base["q"].numel() * base["q"].element_size()

    def make(i):
        if i == 0:
            d = dict(base)
        else:
            d = {n: t.clone() for n, t in base.items()}
        d["out"] = torch.empty_like(d["q"])
        d["wf"] = torch.empty_like(d["w0"])
        return d
    return Rotated(make, per, R_min_bytes)


def bench_linear(B, H, T, d, chunk, loss, dtype, seed, steps, warmup, inp=None, rotate=1 << 30):
    import torch
    import chunked_linear_attention_amd as cla
    import ttt_inputs as ti
    if inp is None:
        inp = ti.gen_linear(B, H, T, T, d, seed=seed, dtype=dtype)
    sets = linear_sets(inp, dtype, rotate)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    nbytes = cla.ttt_linear_workspace_bytes(B, H, T, T, d, chunk, loss, 0, tdt)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device="cuda")

    def call(s):
        cla.ttt_linear_fwd(s["q"], s["k"], s["v"], s["eta"], s["w0"], chunk=chunk, loss=loss,
                           out=s["out"], w_final=s["wf"], workspace=ws)
    ms, med, wall = time_calls(call, sets, steps, warmup)
    esz = 2 if dtype == "bf16" else 4
    NH = B * H
    alg_b = linear_alg_bytes(NH, T, T, d, esz)
    alg_f = linear_alg_flops(NH, T, d, chunk, loss)
    return {"ms": ms, "ms_median": med, "wall_s": wall, "tokens_per_s": B * T / (ms * 1e-3),
            "alg_bytes": alg_b,
            "alg_flops": alg_f, "gbs": alg_b / (ms * 1e-3) / 1e9,
            "tflops": alg_f / (ms * 1e-3) / 1e12, "copies": sets.n}


def lact_alg(NH, Tq, Tkv, d, hid, order):
    flops = NH * (Tkv * 12 * d * hid + Tq * 6 * d * hid)
    byts = NH * (Tkv * (2 * d * 2 + 4) + Tq * 2 * d * 2) + NH * 2 * 3 * d * hid * 4
    return flops, byts


def bench_lact(wl, steps, warmup, rule=None):
    """One LaCT workload.  rule = None (gradient descent through lact_swiglu_fwd)
    or a dict of lact_swiglu_fwd_rule arguments (rule, beta, ns_steps, muon_lr);
    Muon's flops add 4 hid d^2 per matrix and Newton-Schulz step per chunk."""
    import numpy as np
    import torch
    import chunked_linear_attention_amd as cla
    import ttt_inputs as ti
    inp = ti.gen_lact_workload(wl)
    up = lambda n: torch.from_numpy(inp[n + "16"].view(np.int16).copy()).view(torch.bfloat16).cuda()
    s = {n: up(n) for n in ("q", "k", "v")}
    for n in ("eta", "w1", "w2", "w3"):
        s[n] = torch.from_numpy(inp[n]).cuda()
    outs = [torch.empty_like(s["q"]), torch.empty_like(s["w1"]), torch.empty_like(s["w2"]),
            torch.empty_like(s["w3"])]
    nbytes = cla.lact_swiglu_workspace_bytes(wl.B, wl.H, s["q"].shape[2], wl.Tkv, wl.d, wl.hid,
                                             wl.chunk, wl.loss, wl.order, torch.bfloat16)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device="cuda")

    if rule is not None:
        nbytes = cla.lact_swiglu_rule_workspace_bytes(wl.B, wl.H, s["q"].shape[2], wl.Tkv, wl.d,
                                                      wl.hid, wl.chunk, wl.loss, wl.order,
                                                      torch.bfloat16, rule["rule"])
        ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device="cuda")
        mom = [torch.zeros_like(s[n]) for n in ("w1", "w2", "w3")]

    def call(_):
        if rule is None:
            cla.lact_swiglu_fwd(s["q"], s["k"], s["v"], s["eta"], s["w1"], s["w2"], s["w3"],
                                chunk=wl.chunk, loss=wl.loss, order=wl.order,
                                rownorm=bool(wl.rownorm), out=outs[0], w1_final=outs[1],
                                w2_final=outs[2], w3_final=outs[3], workspace=ws)
        else:
            cla.lact_swiglu_fwd_rule(s["q"], s["k"], s["v"], s["eta"], s["w1"], s["w2"], s["w3"],
                                     chunk=wl.chunk, loss=wl.loss, order=wl.order,
                                     rownorm=bool(wl.rownorm), out=outs[0], w1_final=outs[1],
                                     w2_final=outs[2], w3_final=outs[3], workspace=ws,
                                     momentum=mom, **rule)
    class _One:
        def __getitem__(self, i):
            return None
    ms, med, wall = time_calls(call, _One(), steps, warmup)
    NH = wl.B * wl.H
    Tq = s["q"].shape[2]
    flops, byts = lact_alg(NH, Tq, wl.Tkv, wl.d, wl.hid, wl.order)
    name = wl.name
    if rule is not None:
        nchunks = -(-wl.Tkv // wl.chunk)
        if rule["rule"] == "muon":
            flops += NH * nchunks * 3 * rule["ns_steps"] * 4 * wl.hid * wl.d * wl.d
        name += "_" + "_".join(f"{k}{v}" for k, v in rule.items() if k != "rule") + "_" + rule["rule"]
    tok = wl.B * (wl.Tkv if wl.order == 0 else wl.Tkv + Tq)
    return {"workload": name, "ms": ms, "ms_median": med, "steps": steps, "warmup": warmup,
            "tokens_per_s": tok / (ms * 1e-3),
            "tflops": flops / (ms * 1e-3) / 1e12, "mfma_frac": flops / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
            "alg_flops": flops, "alg_bytes": byts}


# ----------------------------------------------------------------------------
# Decode steps (one token per sequence and head; the state is read -- and for
# TTT-Linear rewritten -- once per token).  Algorithmic bytes per head-token:
#   TTT-Linear: state read + write 8 d^2, the chunk-start anchor read 4 d^2
#               (MSE, chunk > 1), the anchor write 4 d^2 once per chunk, q k v
#               and out 4 d s_in, eta 4;
#   LaCT apply: the three weight matrices 12 d hid, q and out 2 d s_in.
# State sets are rotated (>= 1 GiB) so the last-level cache cannot hold them.
def linear_decode_bytes(NH, d, esz, loss, chunk):
    anchored = loss == 1 and chunk > 1
    per = 8 * d * d + (4 * d * d if anchored else 0) + 4 * d * esz + 4
    if chunk > 1:
        per += 4 * d * d / chunk
    return NH * per


def bench_linear_decode(B, H, d, loss, chunk, dtype, steps, warmup, seed=41):
    import numpy as np
    import torch
    import chunked_linear_attention_amd as cla
    import ttt_inputs as ti
    inp = ti.gen_linear(B, H, 1, 1, d, seed=seed, dtype=dtype, w0="normal")
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    if dtype == "bf16":
        up = lambda n: torch.from_numpy(inp[n + "16"][:, :, 0].copy().view(np.int16)).view(torch.bfloat16).cuda()
    else:
        up = lambda n: torch.from_numpy(inp[n][:, :, 0].copy()).cuda()
    q, k, v = up("q"), up("k"), up("v")
    eta = torch.from_numpy(inp["eta"][:, :, 0].copy()).cuda()
    w0 = torch.from_numpy(inp["w0"]).cuda()
    anchored = chunk > 1
    per = w0.numel() * 4 * (2 if anchored else 1)
    sets = Rotated(lambda i: {"w": w0.clone(), "a": w0.clone() if anchored else None}, per,
                   1 << 30, 32)
    out = torch.empty_like(q)
    step = [0]

    def call(s):
        i = step[0]
        step[0] += 1
        cla.ttt_linear_decode(q, k, v, eta, s["w"], loss=loss, w_anchor=s["a"],
                              anchor_update=anchored and i % chunk == chunk - 1, out=out)
    ms, med, _ = time_calls(call, sets, steps, warmup)
    esz = 2 if dtype == "bf16" else 4
    byts = linear_decode_bytes(B * H, d, esz, loss, chunk)
    name = (f"ttt_linear_decode_{'mse' if loss else 'dot'}_B{B}_H{H}_d{d}_"
            f"{'b' + str(chunk) if chunk > 1 else 'recurrent'}_{dtype}")
    return {"workload": name, "us_per_step": ms * 1e3, "us_median": med * 1e3,
            "tokens_per_s": B / (ms * 1e-3), "alg_bytes": byts, "hbm_gbs": byts / (ms * 1e-3) / 1e9,
            "hbm_frac": byts / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, "state_copies": sets.n}


def bench_linear_decode_graph(B, H, d, loss, chunk, replays, seed=41):
    """One chunk of anchored decode steps captured into a HIP graph and replayed:
    the per-step time without host launch overhead.  The state buffers are fixed
    by the capture, so a small batch's state stays in the last-level cache."""
    import numpy as np
    import torch
    import chunked_linear_attention_amd as cla
    import ttt_inputs as ti
    inp = ti.gen_linear(B, H, chunk, chunk, d, seed=seed, dtype="bf16", w0="normal")
    up = lambda n, t: torch.from_numpy(inp[n + "16"][:, :, t].copy().view(np.int16)).view(torch.bfloat16).cuda()
    toks = [(up("q", t), up("k", t), up("v", t), torch.from_numpy(inp["eta"][:, :, t].copy()).cuda())
            for t in range(chunk)]
    w = torch.from_numpy(inp["w0"]).cuda()
    a = w.clone()
    outs = [torch.empty_like(toks[0][0]) for _ in range(chunk)]

    def run():
        for t in range(chunk):
            cla.ttt_linear_decode(*toks[t], w, loss=loss, w_anchor=a, anchor_update=t == chunk - 1,
                                  out=outs[t])
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()

    class _One:
        def __getitem__(self, i):
            return None
    ms, _, _ = time_calls(lambda _: graph.replay(), _One(), replays, 3)
    per = ms / chunk
    return {"workload": f"ttt_linear_decode_{'mse' if loss else 'dot'}_B{B}_H{H}_d{d}_b{chunk}_bf16_graph",
            "us_per_step": per * 1e3, "tokens_per_s": B / (per * 1e-3),
            "note": f"{chunk} steps per graph replay; state resident in the last-level cache"}


def bench_lact_decode(B, H, d, hid, steps, warmup, seed=43):
    import numpy as np
    import torch
    import chunked_linear_attention_amd as cla
    import ttt_inputs as ti
    inp = ti.gen_lact(B, H, 1, 1, d, hid, seed=seed)
    q = torch.from_numpy(inp["q16"][:, :, 0].copy().view(np.int16)).view(torch.bfloat16).cuda()
    ws0 = [torch.from_numpy(inp[n]).cuda() for n in ("w1", "w2", "w3")]
    per = sum(t.numel() * 4 for t in ws0)
    sets = Rotated(lambda i: ws0 if i == 0 else [t.clone() for t in ws0], per, 1 << 30, 32)
    out = torch.empty_like(q)
    nb = cla.lact_swiglu_decode_workspace_bytes(B, H, d, hid, torch.bfloat16)
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")

    def call(s):
        cla.lact_swiglu_decode(q, *s, out=out, workspace=ws)
    ms, med, _ = time_calls(call, sets, steps, warmup)
    byts = B * H * (12 * d * hid + 2 * d * 2)
    return {"workload": f"lact_swiglu_decode_B{B}_H{H}_d{d}_h{hid}_bf16", "us_per_step": ms * 1e3,
            "us_median": med * 1e3,
            "tokens_per_s": B / (ms * 1e-3), "alg_bytes": byts,
            "hbm_gbs": byts / (ms * 1e-3) / 1e9, "hbm_frac": byts / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "state_copies": sets.n}


def bench_decode(steps, warmup):
    """The decode-step workloads: the headline head shape (d = 64, H = 8, MSE,
    chunk-16 anchor) at the headline batch and at a serving batch of 256
    sequences, the recurrent rule, d = 128, and the two LaCT head shapes."""
    res = []
    for args in ((256, 8, 64, 1, 16), (4, 8, 64, 1, 16), (256, 8, 64, 1, 1), (64, 16, 128, 1, 16)):
        log(f"[bench] timing decode {args}")
        res.append(bench_linear_decode(*args, "bf16", steps, warmup))
    log("[bench] timing decode (4, 8, 64, 1, 16) replayed from a graph")
    res.append(bench_linear_decode_graph(4, 8, 64, 1, 16, max(20, steps // 5)))
    for args in ((64, 4, 256, 512), (64, 2, 384, 768)):
        log(f"[bench] timing LaCT decode {args}")
        res.append(bench_lact_decode(*args, steps, warmup))
    return res


def window_attn_flops(NH, T, d, W):
    """2 d flops for each score and 2 d for each value accumulation, per (query,
    key in its window): sum_t min(t + 1, W) keys."""
    pairs = W * (W + 1) // 2 + (T - W) * W if T >= W else T * (T + 1) // 2
    return NH * pairs * 4 * d


def bench_window_attention(B, H, T, d, W, steps, warmup, seed=95):
    import numpy as np
    import torch
    import chunked_linear_attention_amd as cla
    import ttt_inputs as ti
    inp = ti.gen_lact(B, H, T, T, d, 128, seed=seed)
    up = lambda n: torch.from_numpy(inp[n + "16"].view(np.int16).copy()).view(torch.bfloat16).cuda()
    q, k, v = up("q"), up("k"), up("v")
    out = torch.empty_like(q)

    class _One:
        def __getitem__(self, i):
            return None

    ms, med, _ = time_calls(lambda _: cla.window_attention_fwd(q, k, v, window=W, out=out), _One(),
                            steps, warmup)
    fl = window_attn_flops(B * H, T, d, W)
    return {"workload": f"window_attention_B{B}_H{H}_T{T}_d{d}_W{W}_bf16", "ms": ms, "ms_median": med,
            "tokens_per_s": B * T / (ms * 1e-3), "alg_flops": fl,
            "tflops": fl / (ms * 1e-3) / 1e12, "mfma_frac": fl / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS}


def linear_bwd_flops(NH, T, d, b, loss):
    """Per chunk of n tokens: the chunk-start states' forward pass 2nd^2 (MSE:
    +2nd^2) and the adjoints 2nd^2 x (5 inner product | 8 MSE) + 2dn^2 x 4."""
    full, rem = divmod(T, b)
    f = 0
    for n, cnt in ((b, full), (rem, 1 if rem else 0)):
        f += cnt * (2 * n * d * d * ((2 if loss == 1 else 1) + (8 if loss == 1 else 5))
                    + 8 * d * n * n)
    return NH * f


def bench_linear_bwd(B, H, T, d, chunk, loss, steps, warmup, seed=150, order=0):
    import numpy as np
    import torch
    import chunked_linear_attention_amd as cla
    import ttt_inputs as ti
    inp = ti.gen_linear(B, H, T, T, d, seed=seed, dtype="bf16", w0="identity")
    up = lambda a: torch.from_numpy(a.view(np.int16).copy()).view(torch.bfloat16).cuda()
    q, k, v = (up(inp[n + "16"]) for n in ("q", "k", "v"))
    eta, w0 = torch.from_numpy(inp["eta"]).cuda(), torch.from_numpy(inp["w0"]).cuda()
    dy = up(ti.f32_to_bf16_bits(np.random.default_rng(seed).standard_normal(q.shape).astype(np.float32)))
    import chunked_linear_attention_amd._lib as L
    nb = L.load().ttt_linear_bwd_workspace_bytes(B, H, T, T, d, chunk, loss, order, 1)
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")

    class _One:
        def __getitem__(self, i):
            return None

    ms, med, _ = time_calls(lambda _: cla.ttt_linear_bwd(q, k, v, eta, w0, dy, chunk=chunk,
                                                          loss=loss, order=order, workspace=ws),
                            _One(), steps, warmup)
    if order == 1:  # update-then-apply: no intra-chunk terms; reported as time and rate only
        return {"workload": f"ttt_linear_bwd_noncausal_{'mse' if loss else 'dot'}_B{B}_H{H}_T{T}_Tq{T}_d{d}_b{chunk}_bf16",
                "ms": ms, "ms_median": med, "tokens_per_s": B * T / (ms * 1e-3)}
    fl = linear_bwd_flops(B * H, T, d, chunk, loss)
    return {"workload": f"ttt_linear_bwd_{'mse' if loss else 'dot'}_B{B}_H{H}_T{T}_d{d}_b{chunk}_bf16",
            "ms": ms, "ms_median": med, "tokens_per_s": B * T / (ms * 1e-3), "alg_flops": fl,
            "tflops": fl / (ms * 1e-3) / 1e12, "fp32_frac": fl / (ms * 1e-3) / 1e12 / FP32_PEAK_TFLOPS}


def lact_bwd_flops(NH, Tq, Tkv, d, hid):
    """Dense products of the LaCT backward, one per product (the bf16 hi/lo
    pairs multiply the executed count by about 2.5): per key token the replayed
    chunk gradient 12 d hid and the chunk gradient's reverse 30 d hid (H1, H3,
    dG and the three adjoint products over d; three weight adjoints over
    tokens; the key and value adjoints over hidden); per query token the
    apply's reverse 16 d hid."""
    return NH * (Tkv * 42 * d * hid + Tq * 16 * d * hid)


def bench_lact_bwd(wl, steps, warmup, seed=4004):
    """lact_swiglu_bwd on a LaCT workload (upstream gradients of the outputs and
    of the final weights)."""
    import numpy as np
    import torch
    import chunked_linear_attention_amd as cla
    import ttt_inputs as ti
    inp = ti.gen_lact_workload(wl)
    up = lambda a: torch.from_numpy(a.view(np.int16).copy()).view(torch.bfloat16).cuda()
    s = {n: up(inp[n + "16"]) for n in ("q", "k", "v")}
    for n in ("eta", "w1", "w2", "w3"):
        s[n] = torch.from_numpy(inp[n]).cuda()
    rng = np.random.default_rng(seed)
    do = up(ti.f32_to_bf16_bits(rng.standard_normal(inp["q"].shape).astype(np.float32)))
    dw = [torch.from_numpy((0.1 * rng.standard_normal(inp[n].shape)).astype(np.float32)).cuda()
          for n in ("w1", "w2", "w3")]
    Tq = s["q"].shape[2]
    nb = cla.load_library().lact_swiglu_bwd_workspace_bytes(wl.B, wl.H, Tq, wl.Tkv, wl.d, wl.hid,
                                                        wl.chunk, wl.loss, wl.order, 1)
    ws = torch.empty(max(nb, 1), dtype=torch.uint8, device="cuda")

    class _One:
        def __getitem__(self, i):
            return None

    ms, med, _ = time_calls(lambda _: cla.lact_swiglu_bwd(s["q"], s["k"], s["v"], s["eta"], s["w1"],
                                                          s["w2"], s["w3"], do, dw, chunk=wl.chunk,
                                                          order=wl.order, rownorm=bool(wl.rownorm),
                                                          workspace=ws),
                            _One(), steps, warmup)
    NH = wl.B * wl.H
    fl = lact_bwd_flops(NH, Tq, wl.Tkv, wl.d, wl.hid)
    tok = wl.B * (wl.Tkv if wl.order == 0 else wl.Tkv + Tq)
    return {"workload": wl.name + "_bwd", "ms": ms, "ms_median": med, "steps": steps,
            "warmup": warmup, "tokens_per_s": tok / (ms * 1e-3), "alg_flops": fl,
            "tflops": fl / (ms * 1e-3) / 1e12,
            "mfma_frac": fl / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS}


LACT_RULES = ({"rule": "momentum", "beta": 0.9},
              {"rule": "muon", "beta": 0.9, "ns_steps": 5, "muon_lr": 0.02})


def bench_lact_rules(steps, warmup):
    """The causal LaCT workload under the momentum and Muon update rules."""
    out = []
    for r in LACT_RULES:
        log(f"[bench] timing LaCT causal, rule {r}")
        out.append(bench_lact(__import__("ttt_inputs").LACT_CAUSAL, steps, warmup, rule=r))
    return out


def cpu_baseline_linear(inp, chunk, loss, budget_s=10.0, nthreads=0):
    """The oracle as it stands, on the host cores, over whole heads of the workload
    until about `budget_s` of wall time has been spent (at least one call).
    nthreads = 0: every host thread (OpenMP over heads); 1: a single core, on
    as many heads as fit the budget (one head at a time)."""
    import oracle
    B, H, T, d = inp["q"].shape
    NH = B * H
    q = inp["q"].reshape(NH, T, d)
    k = inp["k"].reshape(NH, T, d)
    v = inp["v"].reshape(NH, T, d)
    eta = inp["eta"].reshape(NH, T)
    w0 = inp["w0"].reshape(NH, d, d)
    threads = oracle.max_threads() if nthreads <= 0 else nthreads
    per = NH if threads > 1 else 1   # heads per oracle call
    heads_done, elapsed, h0 = 0, 0.0, 0
    while elapsed < budget_s:
        sl = slice(h0, h0 + per)
        t0 = time.perf_counter()
        oracle.ttt_linear(q[None, sl], k[None, sl], v[None, sl], eta[None, sl], w0[None, sl],
                          chunk=chunk, loss=loss, nthreads=threads)
        elapsed += time.perf_counter() - t0
        heads_done += per
        h0 = (h0 + per) % NH
    how = "OpenMP over heads" if threads > 1 else "one core"
    return {"value": heads_done * T / elapsed, "unit": "tokens/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{heads_done} heads x {T} tokens of the same workload (fp64 token-by-token "
                      f"C oracle, {how}), {elapsed:.1f} s"}


def cpu_baseline_lact(wl, tkv, tq, nthreads=1):
    """The C oracle (fp64 token loop) on a bounded sample of a LaCT workload: one
    head, the first `tkv` update tokens (whole chunks of the workload's chunk size,
    or one chunk of all of them for the non-causal workload) and `tq` queries;
    tokens/s counted like the GPU's (causal: B*T; non-causal: update + query tokens)."""
    import oracle
    import ttt_inputs as ti
    inp = ti.gen_lact_workload(wl, Tkv=tkv, Tq=tq)
    sub = {n: inp[n][:, :1] for n in ("q", "k", "v", "eta", "w1", "w2", "w3")}
    chunk = wl.chunk if wl.order == 0 else tkv
    t0 = time.perf_counter()
    oracle.lact_swiglu(sub["q"], sub["k"], sub["v"], sub["eta"], sub["w1"], sub["w2"], sub["w3"],
                       chunk=chunk, loss=wl.loss, order=wl.order, rownorm=wl.rownorm,
                       nthreads=nthreads)
    el = time.perf_counter() - t0
    tok = tkv if wl.order == 0 else tkv + tq
    return {"workload": wl.name, "value": tok / el, "unit": "tokens/s", "cores": nthreads,
            "kind": "oracle",
            "sample": f"1 head, {tkv} update tokens" + (f" + {tq} queries" if wl.order else "")
                      + f" (chunk {chunk}) of the same workload, fp64 token-by-token C oracle on "
                        f"{nthreads} core(s), {el:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-extras", action="store_true", help="headline workload only")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=10.0)
    ap.add_argument("--lact-only", action="store_true",
                    help="only time the two LaCT workloads (for profiling them alone)")
    ap.add_argument("--bwd-only", action="store_true",
                    help="only time the TTT-Linear backward on the headline shape")
    ap.add_argument("--window-only", action="store_true",
                    help="only time the sliding-window attention workload")
    ap.add_argument("--decode-only", action="store_true",
                    help="only time the decode-step workloads (for profiling them alone)")
    ap.add_argument("--gemm-probe", action="store_true",
                    help="time the LaCT kernels' shared GEMM tile and the vendor GEMM on plain products")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 512 MiB device copy 5 times (scales HBM counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(this library has no multi-GPU path).", file=sys.stderr)
        sys.exit(2)

    import torch
    if args.copy_calibration:
        n = 512 << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        src.fill_(1)
        torch.cuda.synchronize()
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_per_call": n, "calls": 5}))
        return
    import chunked_linear_attention_amd as cla
    import ttt_inputs as ti
    cla.load_library()
    torch.cuda.set_device(0)
    if args.lact_only:
        print(json.dumps({"lact": [bench_lact(lw, args.steps, args.warmup)
                                   for lw in (ti.LACT_CAUSAL, ti.LACT_NONCAUSAL)],
                          "lact_rules": bench_lact_rules(args.steps, args.warmup)}), flush=True)
        return

    if args.gemm_probe:
        print(json.dumps({"gemm_probe": gemm_probe(args.steps, args.warmup)}), flush=True)
        return
    if args.bwd_only:
        # the headline shape, the d = 128 chunk-size sweep's shape, the headline
        # shape in the update-then-apply order, then LaCT
        bwd = [bench_linear_bwd(4, 8, 4096, 64, 16, 1, args.steps, args.warmup)]
        for b in (16, 64, 256, 1024):
            log(f"[bench] TTT-Linear backward B2 H16 T16384 d128 b{b}")
            bwd.append(bench_linear_bwd(2, 16, 16384, 128, b, 1, max(5, args.steps // 10), 2))
        log("[bench] TTT-Linear backward, update-then-apply order, B4 H8 T4096 d64 b16")
        bwd.append(bench_linear_bwd(4, 8, 4096, 64, 16, 1, args.steps, args.warmup, order=1))
        bwd.append(bench_lact_bwd(ti.LACT_CAUSAL, args.steps, args.warmup))
        print(json.dumps({"backward": bwd}), flush=True)
        return
    if args.window_only:
        print(json.dumps({"window_attention": [bench_window_attention(1, 4, 32768, 256, 2048,
                                                                      args.steps, args.warmup)]}),
              flush=True)
        return
    if args.decode_only:
        print(json.dumps({"decode": bench_decode(args.steps, args.warmup)}), flush=True)
        return

    wl = ti.MSE_D64
    seed = ti.WORKLOAD_SEEDS[wl.name]
    log(f"[bench] generating {wl.name}")
    inp = ti.gen_linear_workload(wl)
    log(f"[bench] timing {wl.name}: warmup {args.warmup}, steps {args.steps}")
    r = bench_linear(wl.B, wl.H, wl.T, wl.d, wl.chunk, wl.loss, wl.dtype, seed, args.steps,
                     args.warmup, inp=inp)
    src_hash = kernel_source_hash(["ttt_linear.hip", "ttt_device.h"])
    traffic = read_traffic("ttt_linear", wl.name, src_hash)
    log("[bench] measuring the copy bandwidth and the MFMA-loop rate")
    peaks = measured_peaks()
    line = {
        "metric": METRIC,
        "value": r["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": r["ms"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "batch": wl.B, "heads": wl.H, "seq_len": wl.T,
                   "head_dim": wl.d, "chunk": wl.chunk, "loss": "mse", "order": "causal",
                   "state": "fp32", "input_copies_rotated": r["copies"],
                   "gpu_spin_up_s_before_warmup": SPIN_UP_S},
        "roofline": {"bound": "hbm", "achieved": r["gbs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": r["gbs"] / HBM_PEAK_GBS, "traffic": traffic,
                     "unit_of_launch": "one ttt_linear_fwd call (summary and replay kernels)",
                     "alg_bytes_per_launch": r["alg_bytes"],
                     "kernel_source_sha256_16": src_hash,
                     "ms_median": r["ms_median"],
                     "measured_peak": peaks["hbm_copy_gbs"],
                     "frac_of_measured_peak": r["gbs"] / peaks["hbm_copy_gbs"]},
        "measured_peaks": peaks,
    }
    if not args.no_extras:
        curve = []
        log("[bench] generating the d=128 chunk-sweep workload")
        inp3 = ti.gen_linear_workload(ti.mse_d128(16))
        for b in (16, 64, 256, 1024):
            w3 = ti.mse_d128(b)
            log(f"[bench] timing {w3.name}")
            c = bench_linear(w3.B, w3.H, w3.T, w3.d, b, w3.loss, w3.dtype, 3, EXTRA_STEPS,
                             EXTRA_WARMUP, inp=inp3)
            pages_r = b / (1 + 2 * b / w3.d)
            curve.append({"workload": w3.name, "chunk": b, "tokens_per_s": c["tokens_per_s"],
                          "ms": c["ms"], "ms_median": c["ms_median"], "hbm_gbs": c["gbs"],
                          "hbm_frac": c["gbs"] / HBM_PEAK_GBS,
                          "dual_form_tflops": c["tflops"],
                          "pages_intensity_r_elements": pages_r})
        del inp3
        line["chunk_curve"] = curve
        lact = []
        for lw in (ti.LACT_CAUSAL, ti.LACT_NONCAUSAL):
            try:
                log(f"[bench] timing {lw.name}")
                lact.append(bench_lact(lw, EXTRA_STEPS, EXTRA_WARMUP))
            except Exception as e:  # reported, never hidden
                lact.append({"workload": lw.name, "error": str(e)})
        line["lact"] = lact
        try:
            line["lact_rules"] = bench_lact_rules(EXTRA_STEPS, EXTRA_WARMUP)
        except Exception as e:  # reported, never hidden
            line["lact_rules"] = [{"error": str(e)}]
        line["decode"] = bench_decode(EXTRA_STEPS, EXTRA_WARMUP)
        log("[bench] timing the TTT-Linear backward (headline shape)")
        line["backward"] = [bench_linear_bwd(4, 8, 4096, 64, 16, 1, EXTRA_STEPS, EXTRA_WARMUP)]
        log("[bench] timing the LaCT backward (causal LM workload)")
        try:
            line["backward"].append(bench_lact_bwd(ti.LACT_CAUSAL, 20, 3))
        except Exception as e:  # reported, never hidden
            line["backward"].append({"workload": ti.LACT_CAUSAL.name + "_bwd", "error": str(e)})
        log("[bench] timing the sliding-window attention (LaCT LM shape)")
        line["window_attention"] = [bench_window_attention(1, 4, 32768, 256, 2048, EXTRA_STEPS,
                                                           EXTRA_WARMUP)]
    # every fraction also against the peaks measured in this process
    for c in line.get("chunk_curve", []):
        c["hbm_frac_of_measured"] = c["hbm_gbs"] / peaks["hbm_copy_gbs"]
    for key in ("lact", "lact_rules", "window_attention", "backward"):
        for e in line.get(key, []):
            if "mfma_frac" in e:  # bf16 products (the fp32 TTT-Linear backward has its own fp32_frac)
                e["mfma_frac_of_measured"] = e["tflops"] / peaks["bf16_mfma_tflops"]
    for e in line.get("decode", []):
        if "hbm_gbs" in e:
            e["hbm_frac_of_measured"] = e["hbm_gbs"] / peaks["hbm_copy_gbs"]
    if not args.no_cpu:
        log("[bench] timing the CPU oracle (all host threads, then one core)")
        line["cpu_baseline"] = cpu_baseline_linear(inp, wl.chunk, wl.loss, args.cpu_budget)
        line["cpu_baseline_single_core"] = cpu_baseline_linear(inp, wl.chunk, wl.loss,
                                                               args.cpu_budget, nthreads=1)
        if not args.no_extras:
            log("[bench] timing the CPU oracle on samples of the LaCT workloads (one core)")
            line["cpu_baseline_lact"] = [cpu_baseline_lact(ti.LACT_CAUSAL, 4096, 4096),
                                         cpu_baseline_lact(ti.LACT_NONCAUSAL, 4096, 1024)]
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
