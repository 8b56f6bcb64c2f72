"""Shared helpers for the GPU parity tests: upload seeded inputs, compare to the oracle.

Tolerances (stated once, used everywhere):
* fp32 io: max |delta| <= 2e-3 on the core output o and the norm output y.
* bf16 io: max_i (|delta_i| - s * max(|ref_i|, |gpu_i|))_+ <= 3e-2 * RMS(ref) with
  s = 2^-8 for a call's own output: the bf16 store itself (half an ulp is at most
  2^-8 |x|), which the fp64 oracle does not have; without it no bf16-output
  implementation passes.  A value computed from another bf16 call output (the
  gated norm of the core output o inside a whole-layer check) also carries that
  input's rounding: fp32 and fp64 values of o that straddle a bf16 rounding
  boundary round to neighbours one ulp (<= 2^-7 |o|) apart, which the norm
  passes on element by element, so there s = 2^-8 + 2^-7 = 3 * 2^-8.  (Measured
  with the oracle alone: 1-ulp flips of 1% of o give a gated error of 8e-2 RMS
  at s = 2^-8 and 7e-3 RMS at s = 3 * 2^-8.)
* final recurrent state: per sequence ||dS||_F / ||S_ref||_F <= 1e-3.
* a bf16-stored state: the same Frobenius bound, and element by element
  |a - b| <= 2^-8 (|a| + |b|) + 1e-5 RMS (each side's bf16 store moves a value by
  half an ulp; 1e-5 RMS covers the fp32 arithmetic before it), with a != b on at
  most 1% of the elements.
* conv state: bit-exact (it is a copy of input rows).
"""
from __future__ import annotations

import numpy as np
import torch

F32_ABS_TOL = 2e-3
BF16_RMS_TOL = 3e-2
STATE_REL_TOL = 1e-3
BF16_HALF_ULP = 2.0 ** -8


def to_dev(arr, io: str):
    if arr is None:
        return None
    t = torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32))
    if io == "bf16":
        t = t.to(torch.bfloat16)
    return t.cuda()


def f32_dev(arr):
    return None if arr is None else torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).cuda()


def host(t) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def out_error(gpu, ref, io, upstream_bf16=0):
    """Return (gated error, bound) for an io-dtype output; upstream_bf16 = number of
    bf16 call outputs between the shared inputs and this value (0 or 1)."""
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    assert np.all(np.isfinite(gpu)), "non-finite GPU output"
    d = np.abs(gpu - ref)
    if io == "f32":
        return float(d.max(initial=0.0)), F32_ABS_TOL
    slack = BF16_HALF_ULP * (1 + 2 * upstream_bf16) * np.maximum(np.abs(ref), np.abs(gpu))
    rms = float(np.sqrt(np.mean(ref * ref))) if ref.size else 0.0
    return float(np.maximum(d - slack, 0.0).max(initial=0.0)), BF16_RMS_TOL * rms


def assert_out(gpu, ref, io, what="", upstream_bf16=0):
    err, bound = out_error(gpu, ref, io, upstream_bf16)
    assert err <= bound, f"{what}: error {err:.3e} > bound {bound:.3e} ({io})"
    return err, bound


def assert_state(gpu, ref, what=""):
    """gpu, ref: [..., dk, dv] per (sequence, head); relative Frobenius per leading index 0."""
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert np.all(np.isfinite(gpu)), "non-finite GPU state"
    worst = 0.0
    for s in range(ref.shape[0]):
        den = np.linalg.norm(ref[s])
        num = np.linalg.norm(gpu[s] - ref[s])
        rel = num / den if den > 0 else num
        worst = max(worst, rel)
    assert worst <= STATE_REL_TOL, f"{what}: state rel err {worst:.3e} > {STATE_REL_TOL}"
    return worst


def assert_bf16_state(gpu, ref, what="", max_flip=0.01):
    """gpu, ref: bf16-valued states; equal up to rounding neighbours on few elements.

    Before the bf16 store the two sides differ by the fp32 arithmetic error e of the
    step (taken as 1e-5 RMS(ref), about ten times a 128-term fp32 dot product's); each
    store then moves a value by at most half an ulp, 2^-8 |x|.  So element by element
    |a - b| <= 2^-8 (|a| + |b|) + e, and a and b differ on at most max_flip of them."""
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert_state(gpu, ref, what)
    d = np.abs(gpu - ref)
    e = 1e-5 * float(np.sqrt(np.mean(ref * ref))) if ref.size else 0.0
    excess = d - (BF16_HALF_ULP * (np.abs(gpu) + np.abs(ref)) + e)
    worst = float(excess.max(initial=-1.0))
    assert worst <= 0, f"{what}: a bf16 state element exceeds the rounding bound by {worst:.3e}"
    flips = float(np.mean(d > 0)) if d.size else 0.0
    assert flips <= max_flip, f"{what}: {flips:.2%} of the bf16 state elements differ"
    return flips
