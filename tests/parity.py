"""Helpers shared by the GPU parity tests: move seeded inputs to the GPU, run
the library, run the oracle on the same (rounded) values, compare.

Tolerances (written out here, used by every test):
  fp32 path : max|gpu - oracle| / max|oracle| <= 1e-4        (normwise relative)
  bf16 path : max|gpu - oracle| <= 2e-2 * RMS(oracle)
for outputs and final states.  On top of that the change a call makes is
checked against the oracle's change, so that a mis-scaled update cannot hide
inside the state: W_final - W_init for every path, and for LaCT also
O - f(Q; W_init) (the outputs minus those of the initial weights).

LaCT change bar.  The change is small against the state (about 1-2% of the
weights' RMS per chunk at the workloads' learning rates), and the kernels
hand it bf16 operands (the chunk-start weights, dY, G, dH1, dH3, the
Newton-Schulz iterate and Gram matrix), so bf16 rounding alone moves its
largest element by 1.3-4.2% of its RMS: more than 2e-2 on some inputs, for
any implementation that rounds at these points.  tests/lact_rounding_model.py
computes exactly that floor on the CPU (the method with bf16 roundings at the
kernels' operand points, fp64 elsewhere); on every case measured the GPU's
error equals the model's to two or three digits.  So each LaCT change must
satisfy  error <= max(2e-2, 1.5 x model error)  x RMS(oracle change), the
model error being taken on the same inputs.  For O - f(Q; W_init) each
element is first allowed its own bf16 output rounding (2^-8 |O|), which the
output check already covers and which alone exceeds 2e-2 of the change's RMS
at full size (the change is 7-11% of the outputs' RMS there).
"""
from __future__ import annotations

import numpy as np
import torch

FP32_RTOL = 1e-4
BF16_RMS_TOL = 2e-2
FLOOR_MARGIN = 1.5     # LaCT change bar: max(BF16_RMS_TOL, FLOOR_MARGIN x rounding-model error)


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


def lact_change_errors(got, ref, base, output: bool) -> float:
    """max |got - ref| / RMS(ref - base); for outputs (bf16) each element first
    loses its own rounding allowance 2^-8 |ref|."""
    got, ref, base = (np.asarray(a, dtype=np.float64) for a in (got, ref, base))
    drms = float(np.sqrt(np.mean((ref - base) ** 2)))
    d = np.abs(got - ref)
    if output:
        d = d - np.abs(ref) * 2.0 ** -8
    return float(np.max(d)) / drms if drms > 0 else float(np.max(d))


def assert_lact_change(got, ref, model, base, what: str, output: bool = False):
    """The change check of a LaCT result (see the module docstring).  ``model``
    is the rounding model's result for the same inputs."""
    err = lact_change_errors(got, ref, base, output)
    floor = lact_change_errors(model, ref, base, output)
    bar = max(BF16_RMS_TOL, FLOOR_MARGIN * floor)
    print(f"    {what}: change error {err:.4f}, rounding-model floor {floor:.4f}, bar {bar:.4f}",
          flush=True)
    assert err <= bar, f"{what}: change error {err:.4e} > {bar:.4e} (rounding-model floor {floor:.4e})"


def assert_close_floor(got, ref, model, what: str):
    """2e-2 x RMS like assert_close, unless the rounding model's own error on the
    same inputs exceeds it: then 1.5 x that error.  For LaCT momentum buffers,
    which hold sums of gradients formed from bf16 operands (their value, not
    only their change, sits at the floor the module docstring describes)."""
    got, ref, model = (np.asarray(a, dtype=np.float64) for a in (got, ref, model))
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    rms = float(np.sqrt(np.mean(ref * ref)))
    err = float(np.max(np.abs(got - ref))) / rms
    floor = float(np.max(np.abs(model - ref))) / rms
    bar = max(BF16_RMS_TOL, FLOOR_MARGIN * floor)
    print(f"    {what}: error {err:.4f}, rounding-model floor {floor:.4f}, bar {bar:.4f}", flush=True)
    assert err <= bar, f"{what}: error {err:.4e} > {bar:.4e} x RMS (rounding-model floor {floor:.4e})"
