"""Shared helpers for the GPU parity tests: upload seeded inputs, compare to the oracle.

Tolerances (stated once, used everywhere):
* fp32 io: max |delta| <= 2e-3 on the core output o and the norm output y.
* bf16 io: max_i (|delta_i| - s * max(|ref_i|, |gpu_i|))_+ <= 3e-2 * RMS(ref) with
  s = 2^-8 for a call's own output: the bf16 store itself (half an ulp is at most
  2^-8 |x|), which the fp64 oracle does not have; without it no bf16-output
  implementation passes.  So ref is the oracle's value of that output BEFORE its own
  rounding to bf16 (the oracle rounds a call's output only to feed the next call): a
  rounded reference would add its own half ulp, and wherever the fp32 and fp64 values
  straddle a rounding boundary the two rounded results sit one full ulp apart, which
  at values of several RMS exceeds the bound (measured at full size: 1-ulp flips of
  values near 0.03, nine times the RMS of o).
  Each call is checked on the inputs the GPU gave it (the oracle's core on the GPU's
  conv output, its norm on the GPU's core output).  Checked through the layer instead
  (the oracle's own pipeline from x), a value also carries the rounding of every bf16
  call output upstream of it: fp32 and fp64 values that straddle a bf16 rounding
  boundary round to neighbours one ulp (<= 2^-7 |x|) apart, which the next call passes
  on (the norm element by element; the core through the rows that read the flipped
  element), so there s = 2^-8 (1 + 2 u) for u bf16 call outputs upstream: 3 * 2^-8
  for the core output, 5 * 2^-8 for the norm output.  (Measured with the oracle alone:
  1-ulp flips of 1% of o give a gated error of 8e-2 RMS at s = 2^-8 and 7e-3 RMS at
  s = 3 * 2^-8; at the 397B T=32768 workload, conv-output flips move the core output by
  up to 1.1e-4 at |o| = 0.02 while the core itself, given the GPU's conv output, stays
  within the store's half ulp.)
* final recurrent state: per sequence ||dS||_F / ||S_ref||_F <= 1e-3.
* a bf16-stored state: the same Frobenius bound, and element by element
  |a - b| <= 2^-8 (|a| + |b|) + 1e-5 RMS (each side's bf16 store moves a value by
  half an ulp; 1e-5 RMS covers the fp32 arithmetic before it), with a != b on at
  most 1% of the elements.  A decode step rounds its conv output to bf16 inside the
  call, so the core's k and v carry one bf16 value upstream: where the fp32 and fp64
  conv values straddle a rounding boundary, v_j differs by one ulp and column j of the
  updated state by beta k_i times that ulp (k_c, likewise, moves row c), which is not a
  rounding of the state element itself (measured with the oracle alone, an fp32 conv
  feeding it: 1.0e-4 past that bound at a state RMS of 0.03).  Such a state has the
  element bound on all but 1% of its elements, and the rest within the io outputs'
  3e-2 RMS(ref).
* conv state: bit-exact (it is a copy of input rows).
"""
from __future__ import annotations

import numpy as np

# (torch is imported inside the device helpers only, so that oracle worker processes can
# use the error measures below without it)

F32_ABS_TOL = 2e-3
BF16_RMS_TOL = 3e-2
STATE_REL_TOL = 1e-3
BF16_HALF_ULP = 2.0 ** -8


def to_dev(arr, io: str):
    import torch
    if arr is None:
        return None
    t = torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32))
    if io == "bf16":
        t = t.to(torch.bfloat16)
    return t.cuda()


def f32_dev(arr):
    import torch
    return None if arr is None else torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).cuda()


def host(t) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def excess_stats(gpu, ref, io, upstream_bf16=0):
    """Per-part measures of an io-dtype output that combine over parts of one tensor:
    (largest gated excess, sum of ref^2, element count).  The gated excess is |delta| for
    fp32 io and (|delta| - s max(|ref|, |gpu|))_+ for bf16 io (s as above); the bound on
    the largest excess over the whole tensor uses the RMS of the whole reference."""
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    assert np.all(np.isfinite(gpu)), "non-finite GPU output"
    d = np.abs(gpu - ref)
    if io == "f32":
        ex = float(d.max(initial=0.0))
    else:
        slack = BF16_HALF_ULP * (1 + 2 * upstream_bf16) * np.maximum(np.abs(ref), np.abs(gpu))
        ex = float(np.maximum(d - slack, 0.0).max(initial=0.0))
    return ex, float(np.sum(ref * ref)), int(ref.size)


def bound_of(io, sumsq, count):
    """The error bound of a whole tensor from its reference's sum of squares and size."""
    if io == "f32":
        return F32_ABS_TOL
    return BF16_RMS_TOL * (float(np.sqrt(sumsq / count)) if count else 0.0)


def out_error(gpu, ref, io, upstream_bf16=0):
    """Return (gated error, bound) for an io-dtype output; upstream_bf16 = number of
    bf16 call outputs between the shared inputs and this value (0: a call's own output on
    identical inputs; 1 or 2 through the layer)."""
    ex, sumsq, count = excess_stats(gpu, ref, io, upstream_bf16)
    return ex, bound_of(io, sumsq, count)


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


def assert_bf16_state(gpu, ref, what="", max_flip=0.01, upstream_bf16=0):
    """gpu, ref: bf16-valued states; equal up to rounding neighbours on few elements.

    Before the bf16 store the two sides differ by the fp32 arithmetic error e of the
    step (taken as 1e-5 RMS(ref), about ten times a 128-term fp32 dot product's); each
    store then moves a value by at most half an ulp, 2^-8 |x|.  So element by element
    |a - b| <= 2^-8 (|a| + |b|) + e, and a and b differ on at most max_flip of them.
    upstream_bf16 > 0: the step's k and v were themselves rounded to bf16 (a decode step's
    conv output), and a one-ulp difference there moves a whole row or column of the
    update; then at most max_flip of the elements may pass that bound, each by no more
    than the io outputs' BF16_RMS_TOL RMS(ref)."""
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert_state(gpu, ref, what)
    d = np.abs(gpu - ref)
    rms = float(np.sqrt(np.mean(ref * ref))) if ref.size else 0.0
    excess = d - (BF16_HALF_ULP * (np.abs(gpu) + np.abs(ref)) + 1e-5 * rms)
    worst = float(excess.max(initial=-1.0))
    if upstream_bf16:
        over = float(np.mean(excess > 0)) if d.size else 0.0
        assert over <= max_flip, f"{what}: {over:.2%} of the bf16 state elements exceed the rounding bound"
        assert worst <= BF16_RMS_TOL * rms, \
            f"{what}: a bf16 state element exceeds the rounding bound by {worst:.3e} > {BF16_RMS_TOL} RMS"
    else:
        assert worst <= 0, f"{what}: a bf16 state element exceeds the rounding bound by {worst:.3e}"
    flips = float(np.mean(d > 0)) if d.size else 0.0
    assert flips <= max_flip, f"{what}: {flips:.2%} of the bf16 state elements differ"
    return flips
