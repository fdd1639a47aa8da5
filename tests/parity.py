"""Shared helpers of the GPU parity tests: tolerances and error statistics.

Tolerances (per output tensor, GPU value upcast vs the fp64 oracle, over every
compared element): bf16 outputs max-abs <= 2e-2 and mean-abs <= 2e-3; the
fp32 forward max-abs <= 1e-4; the logsumexp max-abs <= 1e-3.

Grouped key/value heads: dK and dV of a key/value head are the sum of the g
query heads' contributions.  Each contribution is computed exactly as one
ungrouped head (same bound), the contributions' rounding errors come from
independent bf16 roundings of different heads' P and dS and add like
independent noise, and the magnitude of the sum (hence its final bf16
rounding) grows the same way, so the bound on a grouped gradient is the
ungrouped one times sqrt(g).  With g = 1 it is the bound above.
"""
import math
import sys

import numpy as np

BF16_MAX, BF16_MEAN = 2e-2, 2e-3
F32_MAX = 1e-4
LSE_MAX = 1e-3


def grouped(tol, g):
    """Bound on a gradient summed over a group of g query heads."""
    return tol * math.sqrt(g)


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


def check(name, got, ref, max_tol, mean_tol=None):
    mx, mean = errors(got, ref)
    print(f"  [{name}] max_abs={mx:.3e} mean_abs={mean:.3e} (tol max {max_tol:g}"
          + (f", mean {mean_tol:g})" if mean_tol else ")"), flush=True)
    sys.stdout.flush()
    assert mx <= max_tol, f"{name}: max abs error {mx:.3e} > {max_tol:g}"
    if mean_tol is not None:
        assert mean <= mean_tol, f"{name}: mean abs error {mean:.3e} > {mean_tol:g}"
    return mx, mean
