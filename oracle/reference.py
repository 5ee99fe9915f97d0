"""Dequantise-then-matmul definitions (oracle side; test infrastructure only).

What the path computes is ``y = x @ W^T`` for a weight matrix ``W [N, K]`` that
is stored group-quantised. The oracle writes W out in fp64 (exact: every value
is a small integer times an fp16/bf16 scale) and multiplies with BLAS in fp64.

* Ternary weights -- "Kernel experiments: recorded evidence", Test 8 (the CPU
  control reconstructs ``(code - 1) * scale`` in fp64 and multiplies in fp64).
* int8 activations -- same page, Test 6 / Test 7: per 128-group an exact
  integer dot ``P[m,n,g] = sum_k q[m,k] * (code[n,k] - 1)``, then
  ``y = sum_g P * x_scale * w_scale``.
* 4-bit weights with zero points and act-order -- "mate: Marlin-class W4A16
  GEMM for mp_31 (SQMMA int4 x fp16) - #6", conversation and "Act order":
  ``W[n,k] = (code - zero[n, g_idx[k]]) * scale[n, g_idx[k]]`` (the scale is
  indexed through ``g_idx``, not ``k // group``); the permutation sorts the
  K rows by group so that ``x[:, perm] @ W[perm] == x @ W``; a ``g_idx``
  whose sorted groups are not contiguous runs of the group size is refused
  with the invariant named.
* 4-bit weights x int8 activations -- "TensorFold PR #1176" (the int8
  prompt GEMM): per group an exact integer dot of the int8 activations with
  the codes, the weight offset entering through the group's activation sum;
  here the exact partial ``sum q * (code - zero)`` folded like the ternary one.
* 4-bit weights x int8 activations in the page's own form -- "TensorFold PR
  #1176", "What changes": the weight is affine, ``s * code + b`` per group
  (here ``b = -zero * s``), the activations are int8 with one scale ``a``
  and an exact fp32 sum per group, and each group contributes
  ``s * a * (code . q) + b * sum(x)``: the dot on the raw codes 0..15 is
  exact in integers, the offset enters through the sum of the unquantised
  activations.
* Rounded dequantisation for the large-M float path -- the pages' float
  kernels round the dequantised weight to the activation dtype before the
  product ("Kernel experiments", Test 5's batched GEMV; the mate PR's note
  that both kernels unpack int4 to fp16 before the MMA).
"""
from __future__ import annotations

import numpy as np

from . import formats

GROUP = 128


# ---------------------------------------------------------------- act order
def act_order_perm(g_idx: np.ndarray, k: int, group: int = GROUP) -> np.ndarray:
    """Stable argsort of ``g_idx``; refuses malformed group assignments.

    Returns ``perm`` (int64, length K) with ``g_idx[perm[j]] == j // group``.
    """
    g_idx = np.asarray(g_idx)
    if g_idx.shape != (k,):
        raise ValueError(f"g_idx must have shape ({k},), got {g_idx.shape}")
    groups = k // group
    if g_idx.min() < 0 or g_idx.max() >= groups:
        bad = int(np.flatnonzero((g_idx < 0) | (g_idx >= groups))[0])
        raise ValueError(f"g_idx[{bad}] = {int(g_idx[bad])} outside 0..{groups - 1}")
    counts = np.bincount(g_idx.astype(np.int64), minlength=groups)
    wrong = np.flatnonzero(counts != group)
    if wrong.size:
        g = int(wrong[0])
        raise ValueError(f"group {g} has {int(counts[g])} members, expected {group}")
    return np.argsort(g_idx, kind="stable")


# ---------------------------------------------------------------- weights
def weights_ternary(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """codes [N, K] (0..3), scales [N, G] -> W [N, K] fp64 = (code - 1) * scale."""
    n, k = codes.shape
    s = np.asarray(scales, np.float64)
    grp = np.arange(k) // GROUP
    return formats.ternary_value(codes).astype(np.float64) * s[:, grp]


def weights_int4(codes: np.ndarray, scales: np.ndarray, zeros=None, g_idx=None) -> np.ndarray:
    """codes [N, K] (0..15, original K order) -> W [N, K] fp64.

    ``zeros`` None means symmetric codes (value = code - 8). ``g_idx`` None
    means group ``k // 128``.
    """
    n, k = codes.shape
    grp = np.arange(k) // GROUP if g_idx is None else np.asarray(g_idx, np.int64)
    s = np.asarray(scales, np.float64)[:, grp]
    z = 8.0 if zeros is None else np.asarray(zeros, np.float64)[:, grp]
    return (codes.astype(np.float64) - z) * s


def round_to(v: np.ndarray, dtype: str) -> np.ndarray:
    """Round fp64 values to fp16 / bf16 / fp32, nearest-even, returned as fp64.

    Written from the formats' definitions (significand width and the fp16
    subnormal quantum); overflow is not handled because no value here is near
    the top of either range.
    """
    v = np.asarray(v, np.float64)
    if dtype == "f32":
        return v.astype(np.float32).astype(np.float64)
    bits = {"f16": 11, "bf16": 8}[dtype]
    mant, exp = np.frexp(v)                       # v = mant * 2**exp, 0.5 <= |mant| < 1
    quantum_exp = exp - bits
    if dtype == "f16":
        quantum_exp = np.maximum(quantum_exp, -24)   # fp16 subnormal spacing 2**-24
    return np.ldexp(np.rint(np.ldexp(v, -quantum_exp)), quantum_exp)


def weights_int4_rounded(codes, scales, zeros=None, g_idx=None, dtype="bf16") -> np.ndarray:
    """As ``weights_int4`` but each weight rounded to ``dtype`` (the large-M float path)."""
    return round_to(weights_int4(codes, scales, zeros, g_idx), dtype)


# ---------------------------------------------------------------- products
def product(x: np.ndarray, w: np.ndarray) -> np.ndarray:
    """y = x @ W^T in fp64 (BLAS dgemm)."""
    return np.asarray(x, np.float64) @ np.asarray(w, np.float64).T


def ternary_partials(q: np.ndarray, codes: np.ndarray) -> np.ndarray:
    """Exact int group partials P[m, n, g] = sum_{k in g} q[m,k] * (code[n,k] - 1).

    Each group is one fp64 matmul of integers; every partial sum is an integer
    of magnitude below 127 * 2 * 128 < 2**53, so the fp64 result is exact and
    is returned as int64.
    """
    m, k = q.shape
    n = codes.shape[0]
    g = k // GROUP
    qf = q.astype(np.float64).reshape(m, g, GROUP)
    wf = formats.ternary_value(codes).astype(np.float64).reshape(n, g, GROUP)
    out = np.empty((m, n, g), dtype=np.int64)
    for j in range(g):
        out[:, :, j] = (qf[:, j, :] @ wf[:, j, :].T).astype(np.int64)
    return out


def ternary_int8_product(q, x_scale, codes, scales):
    """y[m,n] = x_scale[m] * sum_g w_scale[n,g] * P[m,n,g] (fp64). Returns (P, y)."""
    p = ternary_partials(q, codes)
    s = np.asarray(scales, np.float64)
    y = np.einsum("mng,ng->mn", p.astype(np.float64), s) * np.asarray(x_scale, np.float64)[:, None]
    return p, y


def ternary_int8_product_group_scales(q, x_scale_groups, codes, scales):
    """As above with one activation scale per (row, group): y = sum_g P * xs[m,g] * ws[n,g]."""
    p = ternary_partials(q, codes)
    s = np.asarray(scales, np.float64)
    xs = np.asarray(x_scale_groups, np.float64)
    y = np.einsum("mng,ng,mg->mn", p.astype(np.float64), s, xs)
    return p, y


# ---------------------------------------------------------------- 4-bit x int8
def int4_partials(q: np.ndarray, codes: np.ndarray, zeros=None, g_idx=None) -> np.ndarray:
    """Exact int group partials of 4-bit weights against int8 activations.

    "TensorFold PR #1176" (the int8 prompt GEMM, "What changes"): an affine
    4-bit code is already an exact int8, so each group's dot with int8
    activations is an exact integer, and the weight's offset enters through
    the group's activation sum. With the weights of this library written as
    ``(code - zero) * scale`` the group partial is

        P[m, n, g] = sum over k in group g of q[m, k] * (code[n, k] - zero[n, g])

    with zero = 8 for symmetric codes and group(k) = g_idx[k] under act order,
    else k // 128. Each group is one fp64 matmul of integers below 2**53 in
    magnitude (|P| <= 127 * 15 * 128), so the result is exact; returned as int64.
    """
    m, k = q.shape
    n = codes.shape[0]
    groups = k // GROUP
    grp = np.arange(k) // GROUP if g_idx is None else np.asarray(g_idx, np.int64)
    qf = q.astype(np.float64)
    out = np.empty((m, n, groups), dtype=np.int64)
    for g in range(groups):
        cols = np.flatnonzero(grp == g)
        z = 8.0 if zeros is None else np.asarray(zeros, np.float64)[:, g][:, None]
        wg = codes[:, cols].astype(np.float64) - z
        out[:, :, g] = (qf[:, cols] @ wg.T).astype(np.int64)
    return out


def int4_int8_product(q, x_scale, codes, scales, zeros=None, g_idx=None):
    """y[m,n] = x_scale[m] * sum_g scale[n,g] * P[m,n,g] (fp64), P from ``int4_partials``.

    Returns (P, y). The activation side is int8 with one scale per row, the
    same activation operand as the ternary int8 path.
    """
    p = int4_partials(q, codes, zeros, g_idx)
    s = np.asarray(scales, np.float64)
    y = np.einsum("mng,ng->mn", p.astype(np.float64), s) * np.asarray(x_scale, np.float64)[:, None]
    return p, y


# ------------------------------------------------- 4-bit x int8, affine form
def int4_raw_partials(q: np.ndarray, codes: np.ndarray, g_idx=None) -> np.ndarray:
    """Exact int group dots of the raw 4-bit codes with int8 activations:

        D[m, n, g] = sum over k in group g of q[m, k] * code[n, k],   code in 0..15,

    group(k) = g_idx[k] under act order, else k // 128. |D| <= 127 * 15 * 128 < 2**53,
    so each group's fp64 matmul of integers is exact; returned as int64.
    """
    m, k = q.shape
    n = codes.shape[0]
    groups = k // GROUP
    grp = np.arange(k) // GROUP if g_idx is None else np.asarray(g_idx, np.int64)
    qf = q.astype(np.float64)
    out = np.empty((m, n, groups), dtype=np.int64)
    for g in range(groups):
        cols = np.flatnonzero(grp == g)
        out[:, :, g] = (qf[:, cols] @ codes[:, cols].astype(np.float64).T).astype(np.int64)
    return out


def w4a8_affine_product(q, a, sums, codes, scales, zeros=None, g_idx=None):
    """"TensorFold PR #1176": y[m,n] = sum_g s[n,g] * a[m,g] * D[m,n,g] + b[n,g] * sums[m,g]
    in fp64, with b = -zero * s (zero 8 for symmetric codes) and D from
    ``int4_raw_partials``; a and sums come from the group quantiser with the sums
    (``oracle.quant.quantize_groups_sums``), grouped like the weight. Returns (D, y)."""
    d = int4_raw_partials(q, codes, g_idx)
    s = np.asarray(scales, np.float64)
    z = 8.0 if zeros is None else np.asarray(zeros, np.float64)
    b = -z * s
    af = np.asarray(a, np.float64)
    sf = np.asarray(sums, np.float64)
    y = np.einsum("mng,ng,mg->mn", d.astype(np.float64), s, af) + sf @ b.T
    return d, y
