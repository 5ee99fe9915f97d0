// Activation operand kernels: int8 row and group quantisers, the group
// quantiser with exact group sums (4-bit x int8 in its affine form), int8 plane
// reorder (ternary GEMM), int8 nibble reorder (4-bit x int8 GEMM, with the
// act-order gather), act-order column gather for 16-bit activations.
//
// Quantiser rule: "Kernel experiments: recorded evidence", Test 6 (group-128
// quantiser: absmax / 127, IEEE division, round half to even, clamp to
// +-127) and Test 8 (the division by 127 is a multiply by the fp32 reciprocal).
// Plane order of int8 activations: same page, Test 21 (masked-plane MMA: each
// code plane of a packed byte multiplies a contiguous slice of activations).
// A block (row or group) holding a NaN or an infinity gets scale NaN and
// all-zero codes, so the products that use it come out NaN (the pages say
// nothing of such inputs). The kernels find such values with one fma per
// element, fma(v, 0, acc), which turns NaN exactly when v is NaN or infinite,
// and then take the block's maximum as +inf.
#include "device.h"
#include "launch.h"
#include "qrule.h"

namespace bpw {
namespace {

__device__ __forceinline__ float ld(const float* p) { return *p; }
__device__ __forceinline__ float ld(const __half* p) { return __half2float(*p); }
__device__ __forceinline__ float ld(const uint16_t* p) { return bf16_to_f32(*p); }

constexpr int kQThreads = 256;

// One workgroup per row. ONEPASS (K <= 32 * kQThreads): every value is loaded
// once into registers, the row max is reduced, and the same registers are
// quantised; otherwise the row is read twice.
template <typename T, bool ONEPASS>
__global__ __launch_bounds__(kQThreads) void quantize_rows_kernel(const T* __restrict__ x,
                                                                  int64_t k,
                                                                  int8_t* __restrict__ q,
                                                                  float* __restrict__ x_scale) {
  constexpr int V = 32;
  __shared__ float wmax[kQThreads / 64];
  const int64_t row = blockIdx.x;
  const T* xr = x + row * k;
  int8_t* qr = q + row * k;
  float v[ONEPASS ? V : 1];
  float amax = 0.0f, nonfinite = 0.0f;
  if (ONEPASS) {
#pragma unroll
    for (int j = 0; j < V; ++j) {
      const int64_t i = threadIdx.x + static_cast<int64_t>(j) * kQThreads;
      v[j] = i < k ? ld(xr + i) : 0.0f;
      amax = fmaxf(amax, fabsf(v[j]));
      nonfinite = fmaf(v[j], 0.0f, nonfinite);
    }
  } else {
    for (int64_t i = threadIdx.x; i < k; i += kQThreads) {
      const float x1 = ld(xr + i);
      amax = fmaxf(amax, fabsf(x1));
      nonfinite = fmaf(x1, 0.0f, nonfinite);
    }
  }
  if (nonfinite != nonfinite) amax = __builtin_inff();
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = amax;
  __syncthreads();
  amax = wmax[0];
#pragma unroll
  for (int w = 1; w < kQThreads / 64; ++w) amax = fmaxf(amax, wmax[w]);
  if (__builtin_isinf(amax)) {                      // the whole workgroup takes this branch
    for (int64_t i = threadIdx.x; i < k; i += kQThreads) qr[i] = 0;
    if (threadIdx.x == 0) x_scale[row] = __builtin_nanf("");
    return;
  }
  const float scale = amax * (1.0f / 127.0f);      // fp32 reciprocal constant, one rounding
  const float div = scale > 0.0f ? scale : 1.0f;
  if (ONEPASS) {
#pragma unroll
    for (int j = 0; j < V; ++j) {
      const int64_t i = threadIdx.x + static_cast<int64_t>(j) * kQThreads;
      if (i < k) qr[i] = static_cast<int8_t>(fminf(fmaxf(rintf(v[j] / div), -127.0f), 127.0f));
    }
  } else {
    for (int64_t i = threadIdx.x; i < k; i += kQThreads) {
      float r = rintf(ld(xr + i) / div);             // IEEE division, ties to even
      r = fminf(fmaxf(r, -127.0f), 127.0f);
      qr[i] = static_cast<int8_t>(r);
    }
  }
  if (threadIdx.x == 0) x_scale[row] = scale;
}

// The row quantiser for rows whose K is a multiple of 4 with 4-element-aligned
// vector access: one workgroup of 1024 threads per row, thread t holding the
// 4 elements at 4t + 4096 j (j < V4), so a 4096-column row is one 16-byte (fp32)
// or 8-byte (16-bit) load per thread. The row max is a DPP reduction in each
// wave and a max over the 16 wave maxima through LDS (exact in any order); the
// rule and the non-finite handling are those of quantize_rows_kernel, and each
// thread stores its 4 codes as one 32-bit word.
template <typename T, int V4>
__global__ __launch_bounds__(1024) void quantize_rows_vec_kernel(const T* __restrict__ x, int64_t k,
                                                                 int8_t* __restrict__ q,
                                                                 float* __restrict__ x_scale) {
  __shared__ float wmax[16];
  const int64_t row = blockIdx.x;
  const T* xr = x + row * k;
  int8_t* qr = q + row * k;
  const int tid = threadIdx.x;
  float v[V4][4];
  float amax = 0.0f, nonfinite = 0.0f;
#pragma unroll
  for (int j = 0; j < V4; ++j) {
    const int64_t i = 4 * static_cast<int64_t>(tid) + 4096 * j;
    if (i < k) {
      ld4(xr + i, v[j]);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) v[j][e] = 0.0f;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      amax = fmaxf(amax, fabsf(v[j][e]));
      nonfinite = fmaf(v[j][e], 0.0f, nonfinite);
    }
  }
  if (nonfinite != nonfinite) amax = __builtin_inff();
  amax = wave_max(amax);
  if ((tid & 63) == 0) wmax[tid >> 6] = amax;
  __syncthreads();
  amax = wmax[0];
#pragma unroll
  for (int w = 1; w < 16; ++w) amax = fmaxf(amax, wmax[w]);
  if (__builtin_isinf(amax)) {                      // the whole workgroup takes this branch
#pragma unroll
    for (int j = 0; j < V4; ++j) {
      const int64_t i = 4 * static_cast<int64_t>(tid) + 4096 * j;
      if (i < k) *reinterpret_cast<uint32_t*>(qr + i) = 0u;
    }
    if (tid == 0) x_scale[row] = __builtin_nanf("");
    return;
  }
  const float scale = row_scale(amax);
  const float div = scale > 0.0f ? scale : 1.0f;
#pragma unroll
  for (int j = 0; j < V4; ++j) {
    const int64_t i = 4 * static_cast<int64_t>(tid) + 4096 * j;
    if (i < k) *reinterpret_cast<uint32_t*>(qr + i) = quantize_word(v[j], div);
  }
  if (tid == 0) x_scale[row] = scale;
}

// One wave per (row, 128-group) unit, the same rule with the group's own max:
// unit u covers x[128u, 128u + 128) because rows are K = 128 G long, and its
// scale goes to x_scale[u] ([M][G] row-major). Two values per lane.
template <typename T>
__global__ __launch_bounds__(256) void quantize_groups_kernel(const T* __restrict__ x, int64_t units,
                                                              int8_t* __restrict__ q,
                                                              float* __restrict__ x_scale) {
  const int lane = threadIdx.x & 63;
  for (int64_t u = blockIdx.x * 4ll + (threadIdx.x >> 6); u < units; u += gridDim.x * 4ll) {   // whole waves
    const int64_t i = u * 128 + 2 * lane;
    const float v0 = ld(x + i), v1 = ld(x + i + 1);
    float amax = fmaxf(fabsf(v0), fabsf(v1));
    const float nonfinite = fmaf(v0, 0.0f, v1 * 0.0f);
    if (nonfinite != nonfinite) amax = __builtin_inff();
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
    const bool bad = __builtin_isinf(amax);        // the same in every lane of the wave
    const float scale = bad ? __builtin_nanf("") : amax * (1.0f / 127.0f);   // fp32 reciprocal, one rounding
    const float div = scale > 0.0f ? scale : 1.0f;
    const float r0 = bad ? 0.0f : fminf(fmaxf(rintf(v0 / div), -127.0f), 127.0f);   // IEEE division, ties to even
    const float r1 = bad ? 0.0f : fminf(fmaxf(rintf(v1 / div), -127.0f), 127.0f);
    const uint32_t pair = (static_cast<uint32_t>(static_cast<int>(r0)) & 0xFFu) |
                          ((static_cast<uint32_t>(static_cast<int>(r1)) & 0xFFu) << 8);
    *reinterpret_cast<uint16_t*>(q + i) = static_cast<uint16_t>(pair);
    if (lane == 0) x_scale[u] = scale;
  }
}

// Double-double (hi, lo) arithmetic in fp64 for exact group sums: two_sum
// returns s = fl(a + b) and the exact rounding error e, so a + b == s + e.
__device__ __forceinline__ void two_sum(double a, double b, double& s, double& e) {
  s = a + b;
  const double bb = s - a;
  e = (a - (s - bb)) + (b - bb);
}

// The fp32 value next to finite f, upward (up) or downward, by its bit pattern.
__device__ __forceinline__ float next_f32(float f, bool up) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) == 0) return __uint_as_float(up ? 1u : 0x80000001u);
  const bool away = (static_cast<int32_t>(u) >= 0) == up;              // moving away from zero
  return __uint_as_float(away ? u + 1 : u - 1);
}

// The fp32 nearest (ties to even) to hi + lo, where |lo| <= ulp(hi) / 2. Rounding
// hi alone gives it unless hi is exactly halfway between two fp32 values; then a
// nonzero lo decides the side.
__device__ __forceinline__ float dd_to_f32(double hi, double lo) {
  const float f = static_cast<float>(hi);                         // round to nearest even
  const double df = static_cast<double>(f);
  if (lo == 0.0 || df == hi || !__builtin_isfinite(f)) return f;
  const float g = next_f32(f, hi > df);
  if ((df + static_cast<double>(g)) * 0.5 != hi) return f;      // hi is not a midpoint
  return ((lo > 0.0) == (static_cast<double>(g) > df)) ? g : f;  // the side of hi + lo
}

// "TensorFold PR #1176" (tf_w4a8_quantize): one wave per (row, weight group).
// Group g of a row is the columns perm[128 g .. 128 g + 127] (the identity
// without act order), two per lane. a = fl32(amax / 127) with an IEEE
// division; q = clamp(round_half_even(x / a), -127, 127), written back to its
// own column; the group's sum of x is exact: each lane's two values are added
// with two_sum in fp64, the 64 (hi, lo) pairs are combined in a butterfly of
// two_sum steps (every lane ends with the same pair: each step is symmetric
// in its operands), and the pair is rounded once to fp32. This is exact
// whenever the group's nonzero values span at most 2^73 in magnitude (always
// for fp16 inputs); beyond that the smallest values add with a relative error
// below 2^-104 of the sum. Output pairs (a, sum) go to xs[(row * G + g) * 2].
// A group holding a NaN or an infinity gets a = sum = NaN and zero codes.
// perm entries outside [0, K) read as zero and their code is not written.
template <typename T, bool PERM>
__global__ __launch_bounds__(256) void quantize_groups_sums_kernel(const T* __restrict__ x,
                                                                   const int32_t* __restrict__ perm,
                                                                   int64_t units, int64_t k,
                                                                   int8_t* __restrict__ q,
                                                                   float* __restrict__ xs) {
  const int lane = threadIdx.x & 63;
  const int64_t groups = k >> 7;
  for (int64_t u = blockIdx.x * 4ll + (threadIdx.x >> 6); u < units; u += gridDim.x * 4ll) {   // whole waves
    const int64_t row = u / groups, g = u - row * groups;
    const int64_t j = g * 128 + 2 * lane;
    uint32_t c0 = static_cast<uint32_t>(j), c1 = static_cast<uint32_t>(j + 1);
    if (PERM) {
      c0 = static_cast<uint32_t>(perm[j]);
      c1 = static_cast<uint32_t>(perm[j + 1]);
    }
    const bool in0 = c0 < static_cast<uint64_t>(k), in1 = c1 < static_cast<uint64_t>(k);
    const T* xr = x + row * k;
    const float v0 = in0 ? ld(xr + c0) : 0.0f, v1 = in1 ? ld(xr + c1) : 0.0f;
    float amax = fmaxf(fabsf(v0), fabsf(v1));
    const float nonfinite = fmaf(v0, 0.0f, v1 * 0.0f);
    if (nonfinite != nonfinite) amax = __builtin_inff();
    double hi, lo;
    two_sum(static_cast<double>(v0), static_cast<double>(v1), hi, lo);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      amax = fmaxf(amax, __shfl_xor(amax, off));
      const double ohi = __shfl_xor(hi, off), olo = __shfl_xor(lo, off);
      double sh, se;
      two_sum(hi, ohi, sh, se);
      const double t = (lo + olo) + se;
      hi = sh + t;                                                // fast two_sum: |sh| >= |t|
      lo = t - (hi - sh);
    }
    const bool bad = __builtin_isinf(amax);        // the same in every lane of the wave
    const float a = bad ? __builtin_nanf("") : amax / 127.0f;   // IEEE division
    const float div = a > 0.0f ? a : 1.0f;
    const float r0 = bad ? 0.0f : fminf(fmaxf(rintf(v0 / div), -127.0f), 127.0f);   // ties to even
    const float r1 = bad ? 0.0f : fminf(fmaxf(rintf(v1 / div), -127.0f), 127.0f);
    int8_t* qr = q + row * k;
    if (PERM) {
      if (in0) qr[c0] = static_cast<int8_t>(static_cast<int>(r0));
      if (in1) qr[c1] = static_cast<int8_t>(static_cast<int>(r1));
    } else {
      const uint32_t pair = (static_cast<uint32_t>(static_cast<int>(r0)) & 0xFFu) |
                            ((static_cast<uint32_t>(static_cast<int>(r1)) & 0xFFu) << 8);
      *reinterpret_cast<uint16_t*>(qr + j) = static_cast<uint16_t>(pair);
    }
    if (lane == 0) {
      const float sum = bad ? __builtin_nanf("") : dd_to_f32(hi, lo);
      *reinterpret_cast<float2*>(xs + 2 * u) = float2{a, sum};
    }
  }
}

// One thread per (row, group, half): 64 natural bytes -> four 16-byte plane chunks.
__global__ __launch_bounds__(256) void int8_planes_kernel(const int8_t* __restrict__ q,
                                                          int64_t m, int64_t k,
                                                          int8_t* __restrict__ out) {
  const int64_t units = m * (k / 64);
  for (int64_t u = blockIdx.x * 256ll + threadIdx.x; u < units; u += gridDim.x * 256ll) {
    const int64_t base = u * 64;                     // rows are contiguous: unit u covers [64u, 64u+64)
    const int hh = static_cast<int>(u & 1);
    const v4u* src = reinterpret_cast<const v4u*>(q + base);
    v4u in[4] = {src[0], src[1], src[2], src[3]};
    v4u o[4];
    to_plane_order(in, o);
    int8_t* gbase = out + (base - hh * 64);          // start of the 128-group
#pragma unroll
    for (int t = 0; t < 4; ++t)
      *reinterpret_cast<v4u*>(gbase + 32 * t + 16 * hh) = o[t];
  }
}

// Nibble order for the 4-bit x int8 GEMM, one thread per (row, group, half):
// 64 activation bytes (gathered through perm under act order) -> four 16-byte
// chunks; chunk t holds natural bytes 16t .. 16t + 15 of the half as (even
// bytes of the first 8, odd bytes of the first 8, even and odd of the second 8)
// and goes where plane t of the plane order goes.
__global__ __launch_bounds__(256) void int8_nibbles_kernel(const int8_t* __restrict__ q,
                                                           const int32_t* __restrict__ perm,
                                                           int64_t m, int64_t k,
                                                           int8_t* __restrict__ out) {
  const int64_t per_row = k / 64;
  const int64_t units = m * per_row;
  for (int64_t u = blockIdx.x * 256ll + threadIdx.x; u < units; u += gridDim.x * 256ll) {
    const int64_t base = u * 64;
    const int hh = static_cast<int>(u & 1);
    uint32_t d[16];
    if (perm) {
      const int64_t row = u / per_row;
      const int32_t* pj = perm + (u - row * per_row) * 64;
      const uint8_t* qr = reinterpret_cast<const uint8_t*>(q) + row * k;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        uint32_t v = 0;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const uint32_t c = static_cast<uint32_t>(pj[4 * i + b]);     // out-of-range entries read as 0
          v |= (c < static_cast<uint64_t>(k) ? static_cast<uint32_t>(qr[c]) : 0u) << (8 * b);
        }
        d[i] = v;
      }
    } else {
      const v4u* src = reinterpret_cast<const v4u*>(q + base);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const v4u v = src[i];
        d[4 * i] = v.x;
        d[4 * i + 1] = v.y;
        d[4 * i + 2] = v.z;
        d[4 * i + 3] = v.w;
      }
    }
    int8_t* gbase = out + (base - hh * 64);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const uint32_t* c = d + 4 * t;
      *reinterpret_cast<v4u*>(gbase + 32 * t + 16 * hh) =
          v4u{even_bytes(c[0], c[1]), odd_bytes(c[0], c[1]), even_bytes(c[2], c[3]), odd_bytes(c[2], c[3])};
    }
  }
}

// The same order without act order, one thread per 16-byte chunk: chunk t of
// half h of a 128-group (natural bytes 64h + 16t ..) only moves to offset
// 32t + 16h of the group, with its bytes regrouped as above, so thread j reads
// bytes [16j, 16j + 16) (consecutive threads, consecutive chunks) and writes
// within the same 128-byte group.
__global__ __launch_bounds__(256) void int8_nibbles_chunk_kernel(const int8_t* __restrict__ q, int64_t chunks,
                                                                 int8_t* __restrict__ out) {
  for (int64_t j = blockIdx.x * 256ll + threadIdx.x; j < chunks; j += gridDim.x * 256ll) {
    const v4u c = reinterpret_cast<const v4u*>(q)[j];
    const int t = static_cast<int>(j & 3), hh = static_cast<int>((j >> 2) & 1);
    *reinterpret_cast<v4u*>(out + (j >> 3) * 128 + 32 * t + 16 * hh) =
        v4u{even_bytes(c.x, c.y), odd_bytes(c.x, c.y), even_bytes(c.z, c.w), odd_bytes(c.z, c.w)};
  }
}

__global__ __launch_bounds__(256) void gather_cols_kernel(const uint16_t* __restrict__ x,
                                                          const int32_t* __restrict__ perm,
                                                          int64_t m, int64_t k,
                                                          uint16_t* __restrict__ out) {
  const int64_t total = m * k;
  for (int64_t i = blockIdx.x * 256ll + threadIdx.x; i < total; i += gridDim.x * 256ll) {
    const int64_t row = i / k;
    const int64_t j = i - row * k;
    const uint32_t c = static_cast<uint32_t>(perm[j]);               // out-of-range entries read as 0
    out[i] = c < static_cast<uint64_t>(k) ? x[row * k + c] : static_cast<uint16_t>(0);
  }
}

int grid_for(int64_t items, int per_block) {
  int64_t b = (items + per_block - 1) / per_block;
  if (b > 65536) b = 65536;
  if (b < 1) b = 1;
  return static_cast<int>(b);
}

}  // namespace

template <typename T>
void quantize_go(const void* x, int64_t m, int64_t k, int8_t* q, float* x_scale, hipStream_t s) {
  const size_t va = sizeof(T) * 4;                 // one thread's 4 elements: 16 (fp32) or 8 bytes
  if (k % 4 == 0 && k <= 4 * 4096 && reinterpret_cast<uintptr_t>(x) % va == 0 &&
      reinterpret_cast<uintptr_t>(q) % 4 == 0) {
    const T* xt = static_cast<const T*>(x);
    const dim3 g(static_cast<unsigned>(m));
    switch ((k + 4095) / 4096) {
      case 1: quantize_rows_vec_kernel<T, 1><<<g, 1024, 0, s>>>(xt, k, q, x_scale); break;
      case 2: quantize_rows_vec_kernel<T, 2><<<g, 1024, 0, s>>>(xt, k, q, x_scale); break;
      case 3: quantize_rows_vec_kernel<T, 3><<<g, 1024, 0, s>>>(xt, k, q, x_scale); break;
      default: quantize_rows_vec_kernel<T, 4><<<g, 1024, 0, s>>>(xt, k, q, x_scale); break;
    }
    return;
  }
  dim3 grid(static_cast<unsigned>(m)), block(kQThreads);
  if (k <= 32 * kQThreads)
    quantize_rows_kernel<T, true><<<grid, block, 0, s>>>(static_cast<const T*>(x), k, q, x_scale);
  else
    quantize_rows_kernel<T, false><<<grid, block, 0, s>>>(static_cast<const T*>(x), k, q, x_scale);
}

hipError_t launch_quantize_rows(const void* x, int x_dtype, int64_t m, int64_t k, int8_t* q,
                                float* x_scale, hipStream_t s) {
  switch (x_dtype) {
    case BPW_F32: quantize_go<float>(x, m, k, q, x_scale, s); break;
    case BPW_F16: quantize_go<__half>(x, m, k, q, x_scale, s); break;
    default: quantize_go<uint16_t>(x, m, k, q, x_scale, s); break;
  }
  return hipGetLastError();
}

template <typename T>
void quantize_groups_go(const void* x, int64_t m, int64_t k, int8_t* q, float* x_scale, hipStream_t s) {
  const int64_t units = m * (k / 128);
  quantize_groups_kernel<T><<<grid_for(units, 4), 256, 0, s>>>(static_cast<const T*>(x), units, q, x_scale);
}

hipError_t launch_quantize_groups(const void* x, int x_dtype, int64_t m, int64_t k, int8_t* q,
                                  float* x_scale, hipStream_t s) {
  switch (x_dtype) {
    case BPW_F32: quantize_groups_go<float>(x, m, k, q, x_scale, s); break;
    case BPW_F16: quantize_groups_go<__half>(x, m, k, q, x_scale, s); break;
    default: quantize_groups_go<uint16_t>(x, m, k, q, x_scale, s); break;
  }
  return hipGetLastError();
}

template <typename T>
void quantize_groups_sums_go(const void* x, const int32_t* perm, int64_t m, int64_t k, int8_t* q, float* xs,
                             hipStream_t s) {
  const int64_t units = m * (k / 128);
  if (perm)
    quantize_groups_sums_kernel<T, true><<<grid_for(units, 4), 256, 0, s>>>(static_cast<const T*>(x), perm, units, k,
                                                                           q, xs);
  else
    quantize_groups_sums_kernel<T, false><<<grid_for(units, 4), 256, 0, s>>>(static_cast<const T*>(x), nullptr, units,
                                                                            k, q, xs);
}

hipError_t launch_quantize_groups_sums(const void* x, int x_dtype, const int32_t* perm, int64_t m, int64_t k,
                                       int8_t* q, float* xs, hipStream_t s) {
  switch (x_dtype) {
    case BPW_F32: quantize_groups_sums_go<float>(x, perm, m, k, q, xs, s); break;
    case BPW_F16: quantize_groups_sums_go<__half>(x, perm, m, k, q, xs, s); break;
    default: quantize_groups_sums_go<uint16_t>(x, perm, m, k, q, xs, s); break;
  }
  return hipGetLastError();
}

hipError_t launch_int8_planes(const int8_t* q, int64_t m, int64_t k, int8_t* q_planes,
                              hipStream_t s) {
  const int64_t units = m * (k / 64);
  int8_planes_kernel<<<grid_for(units, 256), 256, 0, s>>>(q, m, k, q_planes);
  return hipGetLastError();
}

hipError_t launch_int8_nibbles(const int8_t* q, const int32_t* perm, int64_t m, int64_t k,
                               int8_t* q_nibbles, hipStream_t s) {
  if (!perm) {
    const int64_t chunks = m * (k / 16);
    int8_nibbles_chunk_kernel<<<grid_for(chunks, 256), 256, 0, s>>>(q, chunks, q_nibbles);
    return hipGetLastError();
  }
  const int64_t units = m * (k / 64);
  int8_nibbles_kernel<<<grid_for(units, 256), 256, 0, s>>>(q, perm, m, k, q_nibbles);
  return hipGetLastError();
}

hipError_t launch_gather_cols(const uint16_t* x, const int32_t* perm, int64_t m, int64_t k,
                              uint16_t* x_perm, hipStream_t s) {
  gather_cols_kernel<<<grid_for(m * k, 256), 256, 0, s>>>(x, perm, m, k, x_perm);
  return hipGetLastError();
}

}  // namespace bpw
