"""int8 activation quantisers (oracle side; test infrastructure only).

"Kernel experiments: recorded evidence", Test 6 (the group-128 quantiser) and
Test 8 (CPU activation-group numerical control):

* ``amax = max |x|`` over the group (fp32),
* ``scale = fl32(amax * fl32(1/127))`` -- the division by the constant 127 is
  a reciprocal multiply in fp32 (Test 8 keeps that rounding on purpose),
* ``q = clamp(round_half_even(fl32(x / scale)), -127, 127)`` with an IEEE
  fp32 division, dividing by 1 instead when the scale is 0 (so q = 0).

The workloads here use one scale per row (``quantize_rows``); the pages' own
granularity is one scale per 128-group (``quantize_groups``).

"TensorFold PR #1176", "What changes" (``quantize_groups_sums``): the int8
prompt path quantises each activation group with one fp32 scale
``a = amax / 127`` (an IEEE fp32 division, not the reciprocal multiply above)
and also records the group's exact fp32 sum of the unquantised activations.
Here the group is the weight's 128-group: the 128 columns ``perm[128 g ..
128 g + 127]`` of the row (``perm`` the weight's act-order permutation, or
the identity), so that ``a`` and the sum pair with the weight group ``g``.
The sum is the exact sum of the group's values rounded once to fp32
(round-to-nearest-even).

Non-finite inputs (the pages are silent): a block holding a NaN or an
infinity gets scale NaN and all-zero codes, so every product output that
uses it comes out NaN instead of a finite value built from the rest.
"""
from __future__ import annotations

import math
from fractions import Fraction

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


def exact_sum_f32(v: np.ndarray) -> np.float32:
    """fp32 rounding (nearest-even) of the exact sum of the finite values ``v``.

    ``math.fsum`` returns the exact sum rounded once to fp64 (s64). Rounding s64 to
    fp32 gives the fp32 rounding of the exact sum, except when s64 is exactly halfway
    between two fp32 values (the exact sum may then lie on either side, or on the
    midpoint itself); that case is settled with the exact rational sum.
    """
    vals = [float(t) for t in np.asarray(v, np.float64).ravel()]
    s64 = math.fsum(vals)
    f = np.float32(s64)
    if float(f) == s64 or not np.isfinite(f):
        return f
    other = np.nextafter(f, np.float32(np.inf) if s64 > float(f) else np.float32(-np.inf))
    if (Fraction(float(f)) + Fraction(float(other))) / 2 != Fraction(s64):
        return f                                   # not a midpoint: s64 and the exact sum round alike
    exact = sum((Fraction(t) for t in vals), Fraction(0))
    mid = Fraction(s64)
    if exact == mid:                               # a true tie: nearest even significand
        return f if int(f.view(np.uint32)) % 2 == 0 else other
    return f if (exact < mid) == (float(f) < s64) else other


def quantize_groups_sums(x: np.ndarray, perm=None, group: int = 128):
    """x [M, K] fp32 -> (q [M, K] int8, a [M, G] fp32, sums [M, G] fp32).

    Group g of row m is the columns perm[group*g : group*(g+1)] (perm None: the
    identity). Per group: a = fl32(amax / 127); q = clamp(round_half_even(fl32(x / a)),
    -127, 127) dividing by 1 when a = 0; sums = the exact sum of the group's x rounded
    once to fp32. q stays in the columns of x. A group holding a NaN or an infinity gets
    a = NaN, sums = NaN and zero codes (as the other quantisers here).
    """
    x = np.asarray(x, dtype=np.float32)
    m, k = x.shape
    g = k // group
    perm = np.arange(k) if perm is None else np.asarray(perm, np.int64)
    xb = x[:, perm].reshape(m, g, group)
    ok = np.isfinite(xb)
    good = ok.all(axis=-1)
    xz = np.where(ok, xb, np.float32(0.0))
    amax = np.max(np.abs(xz), axis=-1)
    a = (amax / np.float32(127.0)).astype(np.float32)          # IEEE fp32 division
    div = np.where(a > 0, a, np.float32(1.0)).astype(np.float32)
    qb = np.clip(np.rint((xz / div[..., None]).astype(np.float32)), -127.0, 127.0)
    qb = np.where(good[..., None], qb, 0.0).astype(np.int8)
    sums = np.empty((m, g), np.float32)
    for i in range(m):
        for j in range(g):
            sums[i, j] = exact_sum_f32(xb[i, j]) if good[i, j] else np.float32(np.nan)
    a = np.where(good, a, np.float32(np.nan)).astype(np.float32)
    q = np.empty((m, k), np.int8)
    q[:, perm] = qb.reshape(m, k)
    return q, a, sums
