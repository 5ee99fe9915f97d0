"""Seeded synthetic inputs for the bit-packed weight path.

This module only draws random numbers and converts storage types. It holds none
of the method's arithmetic: no packing, no quantisation, no dequantisation and
no products. Both the CPU oracle and the GPU path take their inputs from here.

Recipe (one numpy ``default_rng(seed)`` per workload, draws in the order
listed, values drawn in fp64 and then rounded to the storage type):

* ``codes``: one weight code per byte, shape ``[N, K]`` uint8, original K order.
  Ternary: uniform over {0, 1, 2} (meaning -1/0/+1). 4-bit: uniform 0..15.
* ``zeros`` (4-bit with zero points only): uniform 0..15, shape ``[N, G]``.
* ``scales``: uniform over the stated interval, shape ``[N, G]``, rounded to
  fp16 (numpy round-to-nearest-even) or to bf16 (fp64 -> fp32 -> bf16, each
  step round-to-nearest-even; returned as raw uint16 bits).
* ``g_idx`` (act-order only): ``pi = rng.permutation(K)`` then
  ``g_idx[pi[j]] = j // 128``, so each group id owns exactly 128 columns that
  are scattered over K.
* ``x``: standard normal, shape ``[M, K]``, stored as fp32, fp16 or bf16.

G = K / 128 throughout. The five named workloads follow the decode/prefill
shapes used for these weight formats (ternary decode GEMV, W4A16 decode GEMV,
W4A16 prefill GEMM, ternary x int8 prefill GEMM).
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

GROUP = 128


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16, nearest-even, returning the uint16 bit patterns."""
    bits = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    bias = ((bits >> 16) & 1) + 0x7FFF
    return ((bits + bias) >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to fp32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


@dataclasses.dataclass
class Workload:
    """One seeded workload. ``x`` and ``scales`` hold the storage dtype values.

    ``scale_dtype`` / ``x_dtype`` are 'f16', 'bf16' or 'f32'. bf16 arrays hold
    uint16 bit patterns. ``act_int8`` means the activations are meant to be
    quantised to int8 with one scale per row before the product.
    """

    name: str
    fmt: str                 # 'ternary' | 'int4_zp' | 'int4_sym'
    m: int
    k: int
    n: int
    codes: np.ndarray        # [N, K] uint8, one code per byte
    scales: np.ndarray       # [N, G] f16 or bf16 bits
    scale_dtype: str
    x: np.ndarray            # [M, K]
    x_dtype: str
    out_dtype: str           # 'f32' | 'f16' | 'bf16'
    act_int8: bool
    zeros: Optional[np.ndarray] = None   # [N, G] uint8 0..15
    g_idx: Optional[np.ndarray] = None   # [K] int32

    @property
    def groups(self) -> int:
        return self.k // GROUP

    def x_f32(self) -> np.ndarray:
        if self.x_dtype == "bf16":
            return bf16_bits_to_f32(self.x)
        return self.x.astype(np.float32)

    def scales_f64(self) -> np.ndarray:
        if self.scale_dtype == "bf16":
            return bf16_bits_to_f32(self.scales).astype(np.float64)
        return self.scales.astype(np.float64)


def _scales(rng, n, g, lo, hi, dtype):
    s = rng.uniform(lo, hi, size=(n, g))
    if dtype == "f16":
        return s.astype(np.float16)
    return f32_to_bf16_bits(s.astype(np.float32))


def _acts(rng, m, k, dtype):
    x = rng.standard_normal((m, k))
    if dtype == "f32":
        return x.astype(np.float32)
    if dtype == "f16":
        return x.astype(np.float16)
    return f32_to_bf16_bits(x.astype(np.float32))


def ternary_int8(name, seed, m, k, n, scale_lo, scale_hi, out_dtype) -> Workload:
    """Ternary codes {0,1,2}, fp16 group scales, N(0,1) fp32 rows for int8 quantisation."""
    rng = np.random.default_rng(seed)
    g = k // GROUP
    codes = rng.integers(0, 3, size=(n, k), dtype=np.uint8)
    scales = _scales(rng, n, g, scale_lo, scale_hi, "f16")
    x = _acts(rng, m, k, "f32")
    return Workload(name, "ternary", m, k, n, codes, scales, "f16", x, "f32",
                    out_dtype, True)


def int4_zp_actorder(name, seed, m, k, n, scale_lo=0.001, scale_hi=0.02,
                     act_order=True, x_dtype="f16") -> Workload:
    """uint4 codes and zero points, fp16 scales, optional act-order g_idx, fp16 activations."""
    rng = np.random.default_rng(seed)
    g = k // GROUP
    codes = rng.integers(0, 16, size=(n, k), dtype=np.uint8)
    zeros = rng.integers(0, 16, size=(n, g), dtype=np.uint8)
    scales = _scales(rng, n, g, scale_lo, scale_hi, "f16" if x_dtype == "f16" else "bf16")
    g_idx = None
    if act_order:
        pi = rng.permutation(k)
        g_idx = np.empty(k, dtype=np.int32)
        g_idx[pi] = np.arange(k, dtype=np.int32) // GROUP
    x = _acts(rng, m, k, x_dtype)
    return Workload(name, "int4_zp", m, k, n, codes, scales, scales_dtype(x_dtype), x,
                    x_dtype, x_dtype, False, zeros=zeros, g_idx=g_idx)


def scales_dtype(x_dtype):
    return "f16" if x_dtype == "f16" else "bf16"


def int4_sym(name, seed, m, k, n, scale_lo=0.001, scale_hi=0.02, x_dtype="bf16") -> Workload:
    """Symmetric int4 codes (value = code - 8), scales and activations in ``x_dtype``."""
    rng = np.random.default_rng(seed)
    g = k // GROUP
    codes = rng.integers(0, 16, size=(n, k), dtype=np.uint8)
    scales = _scales(rng, n, g, scale_lo, scale_hi, scales_dtype(x_dtype))
    x = _acts(rng, m, k, x_dtype)
    return Workload(name, "int4_sym", m, k, n, codes, scales, scales_dtype(x_dtype), x,
                    x_dtype, x_dtype, False)


# The five named workloads. Seed i-1 for workload i; the M variants of the two
# decode workloads share one draw at the largest M and use its leading rows.
def ternary_tiny() -> Workload:
    return ternary_int8("ternary_gemv_tiny", 0, 1, 512, 256, 0.01, 0.05, "f32")


def ternary_decode(m: int = 1) -> Workload:
    w = ternary_int8("ternary_decode", 1, 16, 4096, 14336, 0.005, 0.05, "f16")
    return leading_rows(w, m)


def w4a16_decode(m: int = 1) -> Workload:
    w = int4_zp_actorder("w4a16_decode", 2, 8, 5120, 13824)
    return leading_rows(w, m)


def w4a16_down(m: int = 1, act_order: bool = True) -> Workload:
    """The down projection paired with the W4A16 decode layer: K and N swapped
    (K=13824, N=5120), the same code, zero-point, scale and activation recipe."""
    w = int4_zp_actorder("w4a16_down", 6, 8, 13824, 5120, act_order=act_order)
    return leading_rows(w, m)


def w4a16_prefill() -> Workload:
    return int4_sym("w4a16_prefill", 3, 2048, 4096, 14336)


def ternary_prefill() -> Workload:
    return ternary_int8("ternary_int8_prefill", 4, 4096, 8192, 28672, 0.005, 0.05, "f16")


def leading_rows(w: Workload, m: int) -> Workload:
    if not 1 <= m <= w.m:
        raise ValueError(f"m={m} outside 1..{w.m}")
    return dataclasses.replace(w, m=m, x=np.ascontiguousarray(w.x[:m]))


NAMED = {
    "ternary_gemv_tiny": ternary_tiny,
    "ternary_decode": ternary_decode,
    "w4a16_decode": w4a16_decode,
    "w4a16_prefill": w4a16_prefill,
    "ternary_int8_prefill": ternary_prefill,
}


def random_int8(seed: int, m: int, k: int) -> np.ndarray:
    """Uniform int8 in [-127, 127] (a stress input for integer partials)."""
    rng = np.random.default_rng(seed)
    return rng.integers(-127, 128, size=(m, k), dtype=np.int8)
