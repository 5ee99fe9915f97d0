"""Parity rule between a GPU output and the fp64 oracle (test infrastructure only).

A product rounded to fp16/bf16 cannot meet an elementwise relative bound of
1e-3 against the unrounded fp64 reference (bf16 alone is up to 2**-8 relative).
The rule: each output must be within 1e-3 (relative, with a floor tau for
results near zero from cancellation) of the reference, plus half a unit in the
last place of the output dtype at the reference value:

    |y - y_ref| <= 1e-3 * max(|y_ref|, tau) + ulp_out(y_ref) / 2,
    tau = 1e-3 * rms(y_ref).

Outputs accumulated in fp32 over K products carry a rounding error that scales
with the sum of the products' magnitudes, not with the result: where the
products cancel (|y_ref| far below tau) no fp32 accumulation meets the floor
above. When the caller passes abs_sum = sum_k |x_k * w_k| for each output (and
K), the bound gains the usual estimate of that error, sqrt(K) * 2**-24 * abs_sum.
"""
from __future__ import annotations

import numpy as np

SIG_BITS = {"f32": 24, "f16": 11, "bf16": 8}
MIN_EXP = {"f32": -126, "f16": -14, "bf16": -126}


def ulp(v: np.ndarray, dtype: str) -> np.ndarray:
    """Spacing of ``dtype`` values at |v|.

    A normal |v| in [2**e, 2**(e+1)) has spacing 2**(e - (p - 1)) for a p-bit
    significand. Zero and the subnormals all have the subnormal quantum
    2**(MIN_EXP - (p - 1)): the binade exponent is clamped to MIN_EXP, and zero
    (for which frexp reports exponent 0) is given MIN_EXP explicitly.
    """
    v = np.abs(np.asarray(v, np.float64))
    _, e = np.frexp(v)                       # v = m * 2**e, 0.5 <= m < 1 (e = 0 for v = 0)
    e = np.where(v == 0.0, MIN_EXP[dtype], np.maximum(e - 1, MIN_EXP[dtype]))
    return np.ldexp(1.0, e - (SIG_BITS[dtype] - 1))


U32 = 2.0 ** -24            # fp32 unit roundoff


def compare(y, y_ref, dtype: str, rel: float = 1e-3, abs_sum=None, k: int = 0) -> dict:
    y = np.asarray(y, np.float64)
    y_ref = np.asarray(y_ref, np.float64)
    if y.shape != y_ref.shape:
        raise ValueError(f"shape {y.shape} != {y_ref.shape}")
    rms = float(np.sqrt(np.mean(y_ref ** 2))) if y_ref.size else 0.0
    tau = rel * rms
    err = np.abs(y - y_ref)
    bound = rel * np.maximum(np.abs(y_ref), tau) + 0.5 * ulp(y_ref, dtype)
    if abs_sum is not None:
        abs_sum = np.asarray(abs_sum, np.float64)
        if abs_sum.shape != y_ref.shape or k < 1:
            raise ValueError("abs_sum must match y_ref's shape and k must be >= 1")
        bound = bound + np.sqrt(k) * U32 * abs_sum
    finite = bool(np.all(np.isfinite(y)))
    denom = np.maximum(np.abs(y_ref), tau if tau > 0 else 1e-300)
    return {
        "ok": finite and bool(np.all(err <= bound)),
        "finite": finite,
        "worst_ratio": float(np.max(err / bound)) if y.size else 0.0,
        "max_rel": float(np.max(err / denom)) if y.size else 0.0,
        "normwise": float(np.max(err) / max(np.max(np.abs(y_ref)), 1e-300)) if y.size else 0.0,
        "rel_rms": float(np.sqrt(np.sum(err ** 2) / max(np.sum(y_ref ** 2), 1e-300))) if y.size else 0.0,
    }
