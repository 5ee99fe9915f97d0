// Device helpers shared by the gfx950 kernels (wave64, MFMA, byte permutes).
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

namespace bpw {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));   // register-friendly (no union)
typedef unsigned v2u __attribute__((ext_vector_type(2)));

// Element-type tags used to instantiate kernels.
struct F32 { typedef float T; };
struct F16 { typedef __half T; };
struct BF16 { typedef uint16_t T; };   // raw bits in memory

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(__half v) { return __half2float(v); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// fp32 -> storage, round to nearest even.
__device__ __forceinline__ void store_out(float* p, float v) { *p = v; }
__device__ __forceinline__ void store_out(__half* p, float v) { *p = __float2half_rn(v); }
__device__ __forceinline__ void store_out(uint16_t* p, float v) {
  __bf16 b = static_cast<__bf16>(v);   // v_cvt_pk_bf16_f32: nearest even
  *p = __builtin_bit_cast(uint16_t, b);
}

// v_perm_b32: byte i of the result is byte sel.byte[i] of the 8-byte value {hi:lo}.
__device__ __forceinline__ uint32_t perm_b32(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}

// (v & mask) | bits in one v_and_or_b32. The mask goes in an SGPR (gfx9 VOP3
// encodings take no literal), bits in a VGPR: the compiler otherwise emits a
// separate AND and OR, each with its literal.
__device__ __forceinline__ uint32_t and_or(uint32_t v, uint32_t mask, uint32_t bits) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(v), "s"(mask), "v"(bits));
  return r;
}

// 4x4 byte transpose: out_t = [i0.byte t, i1.byte t, i2.byte t, i3.byte t].
__device__ __forceinline__ void transpose4x4(uint32_t i0, uint32_t i1, uint32_t i2, uint32_t i3,
                                             uint32_t& o0, uint32_t& o1, uint32_t& o2,
                                             uint32_t& o3) {
  const uint32_t lo01 = perm_b32(i1, i0, 0x05010400u);  // i0.b0 i1.b0 i0.b1 i1.b1
  const uint32_t hi01 = perm_b32(i1, i0, 0x07030602u);  // i0.b2 i1.b2 i0.b3 i1.b3
  const uint32_t lo23 = perm_b32(i3, i2, 0x05010400u);
  const uint32_t hi23 = perm_b32(i3, i2, 0x07030602u);
  o0 = perm_b32(lo23, lo01, 0x05040100u);
  o1 = perm_b32(lo23, lo01, 0x07060302u);
  o2 = perm_b32(hi23, hi01, 0x05040100u);
  o3 = perm_b32(hi23, hi01, 0x07060302u);
}

// 64 activation bytes of one half of a 128-group (natural order, as 16 dwords)
// -> plane order: output chunk t (16 bytes) holds elements 4u + t, u = 0..15.
__device__ __forceinline__ void to_plane_order(const v4u in[4], v4u out[4]) {
  uint32_t d[16] = {in[0].x, in[0].y, in[0].z, in[0].w, in[1].x, in[1].y, in[1].z, in[1].w,
                    in[2].x, in[2].y, in[2].z, in[2].w, in[3].x, in[3].y, in[3].z, in[3].w};
  uint32_t o[4][4];
#pragma unroll
  for (int v = 0; v < 4; ++v)
    transpose4x4(d[4 * v], d[4 * v + 1], d[4 * v + 2], d[4 * v + 3], o[0][v], o[1][v], o[2][v],
                 o[3][v]);
#pragma unroll
  for (int t = 0; t < 4; ++t) out[t] = v4u{o[t][0], o[t][1], o[t][2], o[t][3]};
}

// Sum of the four signed bytes of each dword, accumulated into acc.
__device__ __forceinline__ int sum_i8x4(uint32_t w, int acc) {
  return __builtin_amdgcn_sdot4(static_cast<int>(w), 0x01010101, acc, false);
}

// Ternary code plane t of a packed word: byte j of the result is the code of
// weight 4j + t of the word's four code bytes (values 0..3).
__device__ __forceinline__ uint32_t code_plane(uint32_t w, int t) {
  return (w >> (2 * t)) & 0x03030303u;
}

// Same plane, decoded to signed bytes -1/0/1/2 by a byte select from the table
// {0xff, 0x00, 0x01, 0x02} indexed by the code.
__device__ __forceinline__ uint32_t code_plane_signed(uint32_t w, int t) {
  return perm_b32(0u, 0x020100FFu, code_plane(w, t));
}

// 4-bit codes of one packed dword (byte b: code 2b in the low nibble, code
// 2b + 1 in the high one) as signed bytes code - zero, with zadd holding
// 0x80 - zero in every byte: code + 0x80 - zero stays within 0x71..0x8f (no
// carry into the next byte), and flipping bit 7 gives the two's complement of
// code - zero. nib_lo gives codes 0, 2, 4, 6 of the dword, nib_hi codes 1, 3, 5, 7.
__device__ __forceinline__ uint32_t nib_lo_signed(uint32_t w, uint32_t zadd) {
  return ((w & 0x0F0F0F0Fu) + zadd) ^ 0x80808080u;
}
__device__ __forceinline__ uint32_t nib_hi_signed(uint32_t w, uint32_t zadd) {
  return (((w >> 4) & 0x0F0F0F0Fu) + zadd) ^ 0x80808080u;
}
// The matching activation order: of 8 bytes (a = bytes 0..3, b = bytes 4..7),
// the even ones, then the odd ones.
__device__ __forceinline__ uint32_t even_bytes(uint32_t a, uint32_t b) { return perm_b32(b, a, 0x06040200u); }
__device__ __forceinline__ uint32_t odd_bytes(uint32_t a, uint32_t b) { return perm_b32(b, a, 0x07050301u); }

// Workgroup id remap so that consecutive logical tiles land on the same XCD
// (hardware dispatches workgroup i to XCD i % 8).
__device__ __forceinline__ int xcd_swizzle(int bid, int nblocks) {
  const int per = nblocks / 8;
  const int rem = nblocks % 8;
  const int xcd = bid % 8;
  const int local = bid / 8;
  // XCDs 0..rem-1 own per+1 tiles, the rest own per tiles.
  const int base = xcd < rem ? xcd * (per + 1) : rem * (per + 1) + (xcd - rem) * per;
  return base + local;
}

// Allow a kernel to launch with more than 64 KB of dynamic LDS (gfx950 has 160 KB
// per CU). Called on the host before such a launch; cheap after the first call.
template <typename K>
inline void allow_lds(K* kernel, size_t bytes) {
  if (bytes > 64 * 1024)
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                              hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(bytes));
}

}  // namespace bpw
