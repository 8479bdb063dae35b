"""Error measures and tolerances used by the parity tests.

Softmax family (stable, online streaming, split-row): pure elementwise relative
error max |y - r| / |r|.  No reference element of the workloads underflows, so
the denominator is never zero there; a zero reference element requires an
exact zero.

LayerNorm + GeLU: max |y - r| / max(|r|, 1), i.e. relative error with the
denominator floored at the unit scale of normalized activations.  z = w x_hat + b
cancels near zero, so a pure relative measure would judge rounding noise of
fp32 arithmetic around z = 0, not the kernel.  Where the output is not near
zero the tolerance also holds as a pure relative error: rel_err_above(y, r,
0.01) is max |y - r| / |r| over the elements with |r| >= 0.01.

RMSNorm and fused residual RMSNorm: pure relative error (rel_err), as for
softmax.  y = v * inv_rms * w is a product with no cancellation, and
residual_out = x + residual is one correctly rounded addition; an exact zero
reference (v = 0) demands an exact zero.

Row sums: max_i |y_i - r_i| / sum_j |x_ij|, the error relative to the row's
scale.  A sum may cancel to near zero, where no fp32 summation has a small
relative error; the bound of any summation order is proportional to
sum |x|.  Row max: bit-exact (the max is one of the inputs).

Tolerances: 1e-5 for fp32 input/output, 1e-2 for bf16 storage with fp32
arithmetic.
"""
from __future__ import annotations

import numpy as np

TOL = {"f32": 1e-5, "bf16": 1e-2}


def _arr(a):
    if hasattr(a, "detach"):
        import torch

        a = a.detach().to("cpu", torch.float64).numpy()
    return np.asarray(a, dtype=np.float64)


def rel_err_softmax(y, ref) -> float:
    y, ref = _arr(y), _arr(ref)
    if y.shape != ref.shape:
        raise ValueError(f"shape {y.shape} != {ref.shape}")
    if y.size == 0:
        return 0.0
    if not np.all(np.isfinite(y)):
        return float("inf")
    den = np.abs(ref)
    num = np.abs(y - ref)
    zero = den == 0
    if np.any(num[zero] != 0):
        return float("inf")
    with np.errstate(invalid="ignore", divide="ignore"):
        r = np.where(zero, 0.0, num / np.where(zero, 1.0, den))
    return float(r.max())


def rel_err_floor1(y, ref, floor: float = 1.0) -> float:
    y, ref = _arr(y), _arr(ref)
    if y.shape != ref.shape:
        raise ValueError(f"shape {y.shape} != {ref.shape}")
    if y.size == 0:
        return 0.0
    if not np.all(np.isfinite(y)):
        return float("inf")
    return float((np.abs(y - ref) / np.maximum(np.abs(ref), floor)).max())


def rel_err_above(y, ref, threshold: float) -> float:
    """max |y - r| / |r| over the elements with |r| >= threshold (0 if none)."""
    y, ref = _arr(y), _arr(ref)
    if y.shape != ref.shape:
        raise ValueError(f"shape {y.shape} != {ref.shape}")
    if not np.all(np.isfinite(y)):
        return float("inf")
    sel = np.abs(ref) >= threshold
    if not np.any(sel):
        return 0.0
    return float(np.max(np.abs(y[sel] - ref[sel]) / np.abs(ref[sel])))


def rel_err(y, ref) -> float:
    """max |y - r| / |r| (zero references require exact zeros)."""
    return rel_err_softmax(y, ref)


def rel_err_sum(y, ref, x) -> float:
    """max_i |y_i - r_i| / sum_j |x_ij| over the rows of x."""
    y, ref, x = _arr(y).ravel(), _arr(ref).ravel(), _arr(x)
    if y.shape != ref.shape or x.shape[0] != y.size:
        raise ValueError("shape mismatch")
    if y.size == 0:
        return 0.0
    if not np.all(np.isfinite(y)):
        return float("inf")
    scale = np.abs(x).sum(axis=1)
    num = np.abs(y - ref)
    if np.any(num[scale == 0] != 0):
        return float("inf")
    return float(np.max(np.where(scale == 0, 0.0, num / np.where(scale == 0, 1.0, scale))))
