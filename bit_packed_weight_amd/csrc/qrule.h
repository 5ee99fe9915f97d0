// The int8 row quantiser's rule and the pieces of it that several kernels use:
// "Kernel experiments: recorded evidence", Test 6 (absmax / 127, IEEE
// division, round half to even, clamp to +-127) and Test 8 (the division by
// 127 is a multiply by the fp32 reciprocal). A row holding a NaN or an
// infinity gets scale NaN and all-zero codes; such values are found with one
// fma per element, fma(v, 0, acc), which turns NaN exactly when v is NaN or
// infinite.
#pragma once

#include "device.h"

namespace bpw {

// Max over the 64 lanes of a wave (exact in any order): DPP steps within each
// 16-lane row, then the four row maxima read into scalars.
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false)));
  v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false)));
  v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x141, 0xF, 0xF, false)));
  v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x140, 0xF, 0xF, false)));
  const int vi = __builtin_bit_cast(int, v);
  const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(vi, 0));
  const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(vi, 16));
  const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(vi, 32));
  const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(vi, 48));
  return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

// Four consecutive activations as fp32 (fp32: one 16-byte load; fp16 and bf16:
// one 8-byte load).
__device__ __forceinline__ void ld4(const float* p, float (&v)[4]) {
  const v4f t = *reinterpret_cast<const v4f*>(p);
  v[0] = t.x; v[1] = t.y; v[2] = t.z; v[3] = t.w;
}
__device__ __forceinline__ void ld4(const __half* p, float (&v)[4]) {
  const v2u t = *reinterpret_cast<const v2u*>(p);
  v[0] = __half2float(__builtin_bit_cast(__half, static_cast<uint16_t>(t.x)));
  v[1] = __half2float(__builtin_bit_cast(__half, static_cast<uint16_t>(t.x >> 16)));
  v[2] = __half2float(__builtin_bit_cast(__half, static_cast<uint16_t>(t.y)));
  v[3] = __half2float(__builtin_bit_cast(__half, static_cast<uint16_t>(t.y >> 16)));
}
__device__ __forceinline__ void ld4(const uint16_t* p, float (&v)[4]) {
  const v2u t = *reinterpret_cast<const v2u*>(p);
  v[0] = __uint_as_float(t.x << 16);
  v[1] = __uint_as_float(t.x & 0xFFFF0000u);
  v[2] = __uint_as_float(t.y << 16);
  v[3] = __uint_as_float(t.y & 0xFFFF0000u);
}

// The row scale of a finite absmax: one fp32 multiply by the rounded 1/127.
__device__ __forceinline__ float row_scale(float amax) { return amax * (1.0f / 127.0f); }

// Four codes packed little-endian into a word: rint(v / div) (IEEE division,
// ties to even) clamped to +-127, where div is the row scale or 1 for an
// all-zero row.
__device__ __forceinline__ uint32_t quantize_word(const float (&v)[4], float div) {
  uint32_t word = 0;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float r = fminf(fmaxf(rintf(v[e] / div), -127.0f), 127.0f);
    word |= (static_cast<uint32_t>(static_cast<int>(r)) & 0xFFu) << (8 * e);
  }
  return word;
}

}  // namespace bpw
