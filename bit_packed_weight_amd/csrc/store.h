// Vector output stores shared by the prefill GEMM epilogues.
#pragma once

#include "device.h"

namespace bpw {

// Four consecutive outputs (the address is 4-element aligned), each rounded to
// nearest even as store_out does.
__device__ __forceinline__ void store_out4(float* p, const float (&v)[4]) {
  typedef float v4f __attribute__((ext_vector_type(4)));
  *reinterpret_cast<v4f*>(p) = v4f{v[0], v[1], v[2], v[3]};
}
__device__ __forceinline__ void store_out4(__half* p, const float (&v)[4]) {
  uint32_t w[2];
#pragma unroll
  for (int e = 0; e < 2; ++e)
    w[e] = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, __float2half_rn(v[2 * e]))) |
           (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, __float2half_rn(v[2 * e + 1]))) << 16);
  *reinterpret_cast<v2u*>(p) = v2u{w[0], w[1]};
}
__device__ __forceinline__ void store_out4(uint16_t* p, const float (&v)[4]) {
  uint32_t w[2];
#pragma unroll
  for (int e = 0; e < 2; ++e)
    w[e] = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<__bf16>(v[2 * e]))) |
           (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<__bf16>(v[2 * e + 1]))) << 16);
  *reinterpret_cast<v2u*>(p) = v2u{w[0], w[1]};
}

}  // namespace bpw
