"""int8 activation quantiser (oracle side; test infrastructure only).

"Kernel experiments: recorded evidence", Test 6 (the group-128 quantiser) and
Test 8 (CPU activation-group numerical control):

* ``amax = max |x|`` over the group (fp32),
* ``scale = fl32(amax * fl32(1/127))`` -- the division by the constant 127 is
  a reciprocal multiply in fp32 (Test 8 keeps that rounding on purpose),
* ``q = clamp(round_half_even(fl32(x / scale)), -127, 127)`` with an IEEE
  fp32 division, dividing by 1 instead when the scale is 0 (so q = 0).

The workloads here use one scale per row (``quantize_rows``); the pages' own
granularity is one scale per 128-group (``quantize_groups``).

Non-finite inputs (the pages are silent): a block holding a NaN or an
infinity gets scale NaN and all-zero codes, so every product output that
uses it comes out NaN instead of a finite value built from the rest.
"""
from __future__ import annotations

import numpy as np

INV127 = np.float32(1.0) / np.float32(127.0)


def _quantize_blocks(xb: np.ndarray):
    """xb: [..., L] fp32 -> (q int8 [..., L], scale fp32 [...])."""
    xb = np.asarray(xb, dtype=np.float32)
    ok = np.isfinite(xb)
    good = ok.all(axis=-1)
    xb = np.where(ok, xb, np.float32(0.0))
    amax = np.max(np.abs(xb), axis=-1)
    scale = (amax * INV127).astype(np.float32)
    div = np.where(scale > 0, scale, np.float32(1.0)).astype(np.float32)
    ratio = (xb / div[..., None]).astype(np.float32)      # IEEE fp32 division
    q = np.clip(np.rint(ratio), -127.0, 127.0)            # rint: ties to even
    q = np.where(good[..., None], q, 0.0)
    scale = np.where(good, scale, np.float32(np.nan)).astype(np.float32)
    return q.astype(np.int8), scale


def quantize_rows(x: np.ndarray):
    """x [M, K] fp32 -> (q [M, K] int8, scale [M] fp32), one scale per row."""
    return _quantize_blocks(x)


def quantize_groups(x: np.ndarray, group: int = 128):
    """x [M, K] fp32 -> (q [M, K] int8, scale [M, K/group] fp32)."""
    x = np.asarray(x, dtype=np.float32)
    m, k = x.shape
    q, s = _quantize_blocks(x.reshape(m, k // group, group))
    return q.reshape(m, k), s


def dequantize_rows(q: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """fp64 reconstruction q * scale (per row)."""
    return q.astype(np.float64) * np.asarray(scale, np.float64)[:, None]
