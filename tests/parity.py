"""Helpers shared by the GPU parity tests: move seeded inputs to the GPU, run
the library, run the oracle on the same (rounded) values, compare.

Tolerances (written out here, used by every test):
  fp32 path : max|gpu - oracle| / max|oracle| <= 1e-4        (normwise relative)
  bf16 path : max|gpu - oracle| <= 2e-2 * RMS(oracle)
The same rule is applied to the state change W_final - W_init (against the
oracle's change), so that a mis-scaled update cannot hide inside the state.
For LaCT that change check uses 5e-2 x RMS(change) (DELTA_TOL_LACT): the
change is a sum of products of bf16 operands (dY, G, dH, the bf16 weights) and
its max/RMS ratio is about 5, so one bf16 rounding (relative error up to 2^-8)
per operand already reaches ~2-3% of its RMS at the largest element; a
mis-scaled update, which this check is there to catch, is off by tens of
percent.  W_final itself is held to the 2e-2 x RMS rule.
"""
from __future__ import annotations

import numpy as np
import torch

FP32_RTOL = 1e-4
BF16_RMS_TOL = 2e-2
DELTA_TOL_LACT = 5e-2


def dev(x: np.ndarray, bits: np.ndarray | None = None, dtype=torch.float32) -> torch.Tensor:
    if dtype == torch.bfloat16:
        assert bits is not None
        t = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.cuda()


def inputs_to_device(inp: dict, dtype: str, names=("q", "k", "v")) -> dict:
    out = {}
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    for n in names:
        out[n] = dev(inp[n], inp.get(n + "16"), tdt)
    for n, a in inp.items():
        if n in names or n.endswith("16"):
            continue
        out[n] = dev(a)
    return out


def to_np(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def err_stats(got: np.ndarray, ref: np.ndarray) -> dict:
    diff = np.abs(got - ref)
    rms = float(np.sqrt(np.mean(ref * ref))) if ref.size else 0.0
    mx = float(np.max(np.abs(ref))) if ref.size else 0.0
    md = float(np.max(diff)) if diff.size else 0.0
    return {"max_abs": md, "rms_ref": rms, "max_ref": mx,
            "rel_norm": md / mx if mx > 0 else md, "rel_rms": md / rms if rms > 0 else md,
            "finite": bool(np.all(np.isfinite(got)))}


def assert_close(got: np.ndarray, ref: np.ndarray, dtype: str, what: str, rms_tol=None):
    s = err_stats(got, ref)
    assert s["finite"], f"{what}: non-finite values"
    if ref.size == 0:
        return s
    if dtype == "f32":
        assert s["rel_norm"] <= FP32_RTOL, f"{what}: max rel err {s['rel_norm']:.3e} > {FP32_RTOL} ({s})"
    else:
        tol = BF16_RMS_TOL if rms_tol is None else rms_tol
        assert s["rel_rms"] <= tol, \
            f"{what}: max abs err {s['max_abs']:.3e} > {tol} x RMS {s['rms_ref']:.3e} ({s})"
    return s


def assert_close_bf16_rounded(got: np.ndarray, ref: np.ndarray, what: str, rms_tol=BF16_RMS_TOL):
    """The bf16 rule after allowing each element the rounding of the output itself.

    Used where outputs span a wide range (attention: an early token's output is a
    single value vector, later ones averages with a smaller RMS): rounding the
    exact result to bf16 (nearest even) moves an element by up to half an ulp,
    2^-8 |ref|, which at max|ref| / RMS(ref) > 2.56 alone exceeds 2e-2 x RMS.
    Every element must satisfy |got - ref| <= 2^-8 |ref| + rms_tol x RMS(ref)."""
    s = err_stats(got, ref)
    assert s["finite"], f"{what}: non-finite values"
    excess = np.abs(got - ref) - np.abs(ref) * 2.0 ** -8
    worst = float(np.max(excess)) if excess.size else 0.0
    assert worst <= rms_tol * s["rms_ref"], \
        f"{what}: error beyond output rounding {worst:.3e} > {rms_tol} x RMS {s['rms_ref']:.3e} ({s})"
    return s
