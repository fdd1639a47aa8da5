"""Shared helpers of the GPU parity tests: tolerances and error statistics.

Tolerances (per output tensor, GPU value upcast vs the fp64 oracle, over every
compared element): bf16 outputs max-abs <= 2e-2 and mean-abs <= 2e-3; the
fp32 forward max-abs <= 1e-4; the logsumexp max-abs <= 1e-3.

Gradients summed over a group of query heads (dK, dV of a shared key/value
head): the sum of g heads' contributions can reach magnitudes where a bf16
value's own spacing exceeds the bound (|x| >= 8: half an ulp is 2^-5 > 2e-2),
so even the exact gradient rounded to bf16 would fail a plain 2e-2.  There the
max-abs bound applies to the error beyond that unavoidable output rounding:
per element |got - ref| <= 2e-2 + half a bf16 ulp of ref (check_rounded); the
mean-abs bound is unchanged.  Every other output keeps the plain bounds.

Gradients of attention concentrated on few keys (the drifting-score backward
test): a key that nearly every query attends to sums hundreds of probabilities
near 1, each a bf16 operand of the product, so the operands' own rounding
(half an ulp of 1 is 2^-8) adds up to more than 2e-2.  There each element may
also carry 6 standard deviations of that operand rounding, modelled as
independent and uniform within half an ulp (bf16_rounding_var; check_operand_rounded).
"""
import sys

import numpy as np

BF16_MAX, BF16_MEAN = 2e-2, 2e-3
F32_MAX = 1e-4
LSE_MAX = 1e-3


def to64(t):
    import torch
    return t.detach().to("cpu", torch.float64).numpy()


def errors(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    if got.size == 0:
        return 0.0, 0.0
    if not np.all(np.isfinite(got)):
        return float("inf"), float("inf")
    e = np.abs(got - ref)
    return float(e.max()), float(e.mean())


def bf16_half_ulp(x):
    """Half the spacing of bf16 values around each |x| (8 significant bits):
    2^(floor(log2|x|) - 8); 0 where x is 0."""
    a = np.abs(np.asarray(x, dtype=np.float64))
    out = np.zeros_like(a)
    nz = a > 0
    out[nz] = np.exp2(np.floor(np.log2(a[nz])) - 8)
    return out


def check_rounded(name, got, ref, max_tol=BF16_MAX, mean_tol=BF16_MEAN):
    """Bound for bf16 outputs that may exceed the magnitude where their own
    rounding fits the max-abs bound: every element within max_tol plus half a
    bf16 ulp of the reference value, and the mean-abs bound as usual.  Prints
    the plain max-abs error beside the error of the exact value rounded to
    bf16 (the best any bf16 output can do)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    if got.size == 0:
        return 0.0, 0.0
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    import torch
    e = np.abs(got - ref)
    best = np.abs(torch.from_numpy(ref).to(torch.bfloat16).double().numpy() - ref).max()
    excess = float((e - bf16_half_ulp(ref)).max())
    mx, mean = float(e.max()), float(e.mean())
    print(f"  [{name}] max_abs={mx:.3e} (exact value rounded to bf16: {best:.3e}) "
          f"max beyond half an ulp={excess:.3e} mean_abs={mean:.3e} (tol {max_tol:g} + half ulp, mean {mean_tol:g})",
          flush=True)
    assert excess <= max_tol, f"{name}: error beyond half a bf16 ulp {excess:.3e} > {max_tol:g}"
    assert mean <= mean_tol, f"{name}: mean abs error {mean:.3e} > {mean_tol:g}"
    return mx, mean


def check(name, got, ref, max_tol, mean_tol=None):
    mx, mean = errors(got, ref)
    print(f"  [{name}] max_abs={mx:.3e} mean_abs={mean:.3e} (tol max {max_tol:g}"
          + (f", mean {mean_tol:g})" if mean_tol else ")"), flush=True)
    sys.stdout.flush()
    assert mx <= max_tol, f"{name}: max abs error {mx:.3e} > {max_tol:g}"
    if mean_tol is not None:
        assert mean <= mean_tol, f"{name}: mean abs error {mean:.3e} > {mean_tol:g}"
    return mx, mean


def bf16_rounding_var(x):
    """Variance of rounding each element of x to bf16 (RNE), modelled as
    uniform within half an ulp: ulp^2 / 12 with ulp = 2^(floor(log2|x|) - 7)."""
    a = np.abs(np.asarray(x, dtype=np.float64))
    out = np.zeros_like(a)
    nz = a > 0
    out[nz] = np.exp2(2 * (np.floor(np.log2(a[nz])) - 7)) / 12.0
    return out


def check_operand_rounded(name, got, ref, sigma, max_tol=BF16_MAX, mean_tol=BF16_MEAN, k=6.0):
    """Per element |got - ref| <= max_tol + half a bf16 ulp of ref + k·sigma,
    sigma the standard deviation the bf16 rounding of the products' operands
    implies for that element; the mean-abs bound as usual."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    sigma = np.asarray(sigma, dtype=np.float64)
    assert got.shape == ref.shape == sigma.shape, (got.shape, ref.shape, sigma.shape)
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    e = np.abs(got - ref)
    excess = e - bf16_half_ulp(ref) - k * sigma
    mx, mean = float(e.max()), float(e.mean())
    print(f"  [{name}] max_abs={mx:.3e} max beyond half an ulp and {k:g} sigma={float(excess.max()):.3e} "
          f"(largest sigma {float(sigma.max()):.3e}) mean_abs={mean:.3e} (tol {max_tol:g}, mean {mean_tol:g})",
          flush=True)
    assert float(excess.max()) <= max_tol, f"{name}: error beyond rounding {float(excess.max()):.3e} > {max_tol:g}"
    assert mean <= mean_tol, f"{name}: mean abs error {mean:.3e} > {mean_tol:g}"
    return mx, mean
