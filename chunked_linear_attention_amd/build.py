"""Build libttt_mi355x.so (gfx950 only) in-tree with hipcc.

Each translation unit under csrc/ is compiled to an object in _build/ and the
objects are linked into chunked_linear_attention_amd/libttt_mi355x.so.  The
build always recompiles (it is also the "does it build" check).
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libttt_mi355x.so")
# (source, object name, extra flags): the TTT-Linear backward is compiled
# twice, its multi-tile path as a unit of its own (see FLAGS)
SOURCES = [("api.cpp", "api", []), ("ttt_linear.hip", "ttt_linear", []), ("lact_swiglu.hip", "lact_swiglu", []),
           ("decode.hip", "decode", []), ("window_attn.hip", "window_attn", []),
           ("ttt_linear_bwd.hip", "ttt_linear_bwd", []),
           ("ttt_linear_bwd.hip", "ttt_linear_bwd_tiled", ["-DTTT_LBW_TILED_UNIT"]),
           ("probe.hip", "probe", []), ("noalloc.hip", "noalloc", []), ("lact_swiglu_bwd.hip", "lact_swiglu_bwd", [])]

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
COMMON = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
          # keep packed fp32 instructions out of the generated code
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I", os.path.join(ROOT, "include"), "-I", CSRC]
# Per-source flags: MFMA operands and results forced into VGPRs (no
# AGPR<->VGPR copies around the vector work between products).  Measured
# against the compiler's own choice in one process (library variants timed
# back to back): TTT-Linear keeps it (its state sits in MFMA accumulators that
# the vector code updates); the LaCT forward gained ~4% on the causal and ~2%
# on the non-causal workload with it; the LaCT backward, once its GEMM no
# longer held its segment pointers in registers, gained ~1.6% (9.61 -> 9.46 ms;
# before that change it was ~1% slower with the flag); the TTT-Linear
# backward's multi-tile path is 3-18% faster with it across chunk sizes 32 to
# 1024 at d = 64 and 128, its 16-token path 2-4% slower (so only the former's
# unit takes it).  Keyed by object name.
FLAGS = {"ttt_linear": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
         "lact_swiglu": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
         "lact_swiglu_bwd": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
         "ttt_linear_bwd_tiled": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _compile(entry) -> str:
    src, name, extra = entry
    obj = os.path.join(BUILD, name + ".o")
    lang = ["-x", "hip"] if src.endswith(".cpp") else []
    cmd = [HIPCC] + COMMON + FLAGS.get(name, []) + extra + lang + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed on {src}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("link failed")
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
