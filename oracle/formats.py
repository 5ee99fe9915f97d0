"""Bit layouts of the packed weights (oracle side; test infrastructure only).

Ternary ("PQ2") format -- "Kernel experiments: recorded evidence", section A
(Diagram 1, Test 1 and Test 2): 128 weights share one fp16 scale; each byte
holds four 2-bit codes; a weight's value is its code minus one. Within a
128-group, code byte j carries weights 4j..4j+3, weight 4j+t in bits 2t..2t+1
(Test 2's byte-expanded MMQ reshapes byte x plane into the 128-wide dot in
exactly this order). A raw block is 34 bytes: the fp16 scale (little-endian)
then the 32 code bytes (Test 8's CPU control reads blocks this way).

4-bit formats -- "mate: Marlin-class W4A16 GEMM for mp_31 (SQMMA int4 x fp16)
- #6": int4 codes with one scale (and optionally one zero point) per group.
The pages do not fix the nibble order; this oracle reads the low nibble as the
even K index (and, for zero points, the even group index).
"""
from __future__ import annotations

import numpy as np

GROUP = 128
PQ2_BLOCK = 34


def ternary_value(codes: np.ndarray) -> np.ndarray:
    """Signed weight value of a 2-bit code: code - 1 (code 3 decodes to +2)."""
    return codes.astype(np.int64) - 1


def unpack_ternary(plane: np.ndarray, k: int) -> np.ndarray:
    """Code plane ``[N, K/4]`` uint8 -> codes ``[N, K]`` (0..3), K in original order."""
    plane = np.asarray(plane, dtype=np.uint8)
    n = plane.shape[0]
    if plane.shape[1] * 4 != k:
        raise ValueError("ternary plane must hold K/4 bytes per row")
    shifts = np.arange(4, dtype=np.uint8) * 2
    codes = (plane[:, :, None] >> shifts[None, None, :]) & 3   # [N, K/4, 4]: weight 4*byte + t
    return codes.reshape(n, k).astype(np.uint8)


def pack_ternary(codes: np.ndarray) -> np.ndarray:
    """Codes ``[N, K]`` (0..3) -> code plane ``[N, K/4]`` (inverse of ``unpack_ternary``)."""
    codes = np.asarray(codes, dtype=np.uint8)
    n, k = codes.shape
    c = codes.reshape(n, k // 4, 4).astype(np.uint32)
    out = c[:, :, 0] | (c[:, :, 1] << 2) | (c[:, :, 2] << 4) | (c[:, :, 3] << 6)
    return out.astype(np.uint8)


def split_pq2_blocks(raw: np.ndarray):
    """Raw PQ2 rows ``[N, G*34]`` -> (code plane ``[N, K/4]``, fp16 scales ``[N, G]``)."""
    raw = np.asarray(raw, dtype=np.uint8)
    n, width = raw.shape
    if width % PQ2_BLOCK:
        raise ValueError("PQ2 row width must be a multiple of 34")
    blocks = raw.reshape(n, width // PQ2_BLOCK, PQ2_BLOCK)
    scales = np.ascontiguousarray(blocks[:, :, :2]).view("<f2").reshape(n, width // PQ2_BLOCK)
    plane = np.ascontiguousarray(blocks[:, :, 2:]).reshape(n, width // PQ2_BLOCK * 32)
    return plane, scales.astype(np.float16)


def join_pq2_blocks(plane: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Inverse of ``split_pq2_blocks``."""
    n = plane.shape[0]
    g = scales.shape[1]
    blocks = np.empty((n, g, PQ2_BLOCK), dtype=np.uint8)
    blocks[:, :, :2] = np.ascontiguousarray(scales.astype("<f2")).view(np.uint8).reshape(n, g, 2)
    blocks[:, :, 2:] = plane.reshape(n, g, 32)
    return blocks.reshape(n, g * PQ2_BLOCK)


def unpack_int4(plane: np.ndarray, k: int) -> np.ndarray:
    """4-bit plane ``[N, K/2]`` -> codes ``[N, K]`` (0..15); low nibble = even K index."""
    plane = np.asarray(plane, dtype=np.uint8)
    n = plane.shape[0]
    if plane.shape[1] * 2 != k:
        raise ValueError("4-bit plane must hold K/2 bytes per row")
    lo = plane & 0x0F
    hi = plane >> 4
    return np.stack([lo, hi], axis=2).reshape(n, k).astype(np.uint8)


def pack_int4(codes: np.ndarray) -> np.ndarray:
    """Codes ``[N, K]`` (0..15) -> plane ``[N, K/2]`` (inverse of ``unpack_int4``)."""
    codes = np.asarray(codes, dtype=np.uint8)
    n, k = codes.shape
    c = codes.reshape(n, k // 2, 2)
    return (c[:, :, 0] | (c[:, :, 1] << 4)).astype(np.uint8)


def unpack_zeros(zplane: np.ndarray, groups: int) -> np.ndarray:
    """Zero-point plane ``[N, ceil(G/2)]`` -> zeros ``[N, G]``; low nibble = even group."""
    z = unpack_int4(zplane, zplane.shape[1] * 2)
    return z[:, :groups]


def pack_zeros(zeros: np.ndarray) -> np.ndarray:
    zeros = np.asarray(zeros, dtype=np.uint8)
    n, g = zeros.shape
    if g % 2:
        zeros = np.concatenate([zeros, np.zeros((n, 1), np.uint8)], axis=1)
    return pack_int4(zeros)
