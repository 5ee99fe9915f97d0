// Decode-shaped products (M <= 32) on gfx950 MFMA.
//
// Workgroup = one tile of 32 weight rows; its NW waves split K into contiguous
// group ranges; the activations of all M rows are staged once into LDS in the
// order the matrix instruction reads them; the per-wave fp32 partials are summed
// across waves in a fixed order. Each weight byte is read from HBM exactly once,
// with 16-byte loads (two lanes cover one 32-byte ternary group of a row, four
// 16-byte loads cover one 64-byte 4-bit group).
//
// Ternary x int8 -- "Kernel experiments: recorded evidence", Test 6 (integer
// group dots, fp32 scale fold) and Test 21 (code planes of a packed byte
// multiply plane-ordered activations; the code - 1 offset is applied once per
// group as minus the group sum of q). MFMA i32_32x32x32_i8: A = activations
// (row = token), B = code planes (column = weight row).
//
// 4-bit x fp16/bf16 -- "mate: Marlin-class W4A16 GEMM for mp_31 (SQMMA int4 x
// fp16) - #6": a decode GEMV that reads each weight once; the zero point is
// subtracted from the code exactly (code - zero is an integer in -15..15) and
// the group scale is applied to the fp32 group partial.
#include "device.h"
#include "launch.h"

namespace bpw {
namespace {

constexpr int kRows = 32;                    // weight rows per workgroup (MFMA width)
constexpr size_t kLdsBudget = 128 * 1024;    // staged activations per workgroup
constexpr int kMaxG = 8;                     // groups kept in flight per wave

// D layout of a 32x32 MFMA: lane l holds column l % 32 and rows
// 8*(r/4) + 4*(l/32) + r%4 for its 16 accumulator registers r.
__device__ __forceinline__ int d_row(int r, int h) { return 8 * (r >> 2) + 4 * h + (r & 3); }

template <int NW, int FOLD, typename TOut, bool PARTIALS>
__global__ __launch_bounds__(NW * 64) void gemv_t2_kernel(
    const uint8_t* __restrict__ codes, const __half* __restrict__ wscale,
    const int8_t* __restrict__ q, const float* __restrict__ x_scale, int M, int N, int K,
    TOut* __restrict__ y, int32_t* __restrict__ pout, int pm0, int pm1, int pn0, int pn1,
    int tile0) {
  extern __shared__ __align__(16) uint8_t smem[];
  const int G = K >> 7;
  const int KB = K >> 2;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n0 = (blockIdx.x + tile0) * kRows;
  uint8_t* qs = smem;                                            // [M][K] plane order
  int* ts = reinterpret_cast<int*>(smem + static_cast<size_t>(M) * K);   // [M][G] group sums

  const int gpw = (G + NW - 1) / NW;
  const int gb = min(G, wave * gpw);
  const int ge = min(G, gb + gpw);
  const int n = lane & 31, h = lane >> 5;
  const int row = min(n0 + n, N - 1);
  const uint8_t* crow = codes + static_cast<size_t>(row) * KB + h * 16;
  const __half* srow = wscale + static_cast<size_t>(row) * G;

  // Issue this wave's first weight loads before staging the activations.
  uint4 cw[kMaxG];
  float sc[kMaxG];
#pragma unroll
  for (int u = 0; u < kMaxG; ++u) {
    if (gb + u < ge) {
      cw[u] = *reinterpret_cast<const uint4*>(crow + static_cast<size_t>(gb + u) * 32);
      sc[u] = __half2float(srow[gb + u]);
    }
  }

  // Stage q into plane order and compute exact group sums.
  const int units = M * G * 2;
  for (int u = tid; u < units; u += NW * 64) {
    const int hh = u & 1, mg = u >> 1;
    const int m = mg / G, g = mg - m * G;
    const uint4* src = reinterpret_cast<const uint4*>(q + static_cast<size_t>(m) * K + g * 128 + hh * 64);
    uint4 in[4] = {src[0], src[1], src[2], src[3]};
    uint4 o[4];
    to_plane_order(in, o);
    uint8_t* dst = qs + static_cast<size_t>(m) * K + g * 128 + hh * 16;
#pragma unroll
    for (int t = 0; t < 4; ++t) *reinterpret_cast<uint4*>(dst + 32 * t) = o[t];
    int sum = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sum = sum_i8x4(in[i].x, sum);
      sum = sum_i8x4(in[i].y, sum);
      sum = sum_i8x4(in[i].z, sum);
      sum = sum_i8x4(in[i].w, sum);
    }
    sum += __shfl_xor(sum, 1);
    if (hh == 0) ts[m * G + g] = sum;
  }
  __syncthreads();

  const int mA = min(n, M - 1);
  const uint8_t* qa = qs + static_cast<size_t>(mA) * K + h * 16;
  float acc[FOLD];
#pragma unroll
  for (int r = 0; r < FOLD; ++r) acc[r] = 0.0f;

  for (int g0 = gb; g0 < ge; g0 += kMaxG) {
    if (g0 != gb) {
#pragma unroll
      for (int u = 0; u < kMaxG; ++u) {
        if (g0 + u < ge) {
          cw[u] = *reinterpret_cast<const uint4*>(crow + static_cast<size_t>(g0 + u) * 32);
          sc[u] = __half2float(srow[g0 + u]);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kMaxG; ++u) {
      const int g = g0 + u;
      if (g < ge) {
        v16i d = {};
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const v4i b = {static_cast<int>(code_plane(cw[u].x, t)), static_cast<int>(code_plane(cw[u].y, t)),
                         static_cast<int>(code_plane(cw[u].z, t)), static_cast<int>(code_plane(cw[u].w, t))};
          const v4i a = *reinterpret_cast<const v4i*>(qa + g * 128 + 32 * t);
          d = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, d, 0, 0, 0);
        }
        if (PARTIALS) {
          const int nn = n0 + n;
#pragma unroll
          for (int r = 0; r < FOLD; ++r) {
            const int mm = d_row(r, h);
            if (mm >= pm0 && mm < pm1 && nn >= pn0 && nn < pn1) {
              const int p = d[r] - ts[mm * G + g];
              pout[(static_cast<size_t>(mm - pm0) * (pn1 - pn0) + (nn - pn0)) * G + g] = p;
            }
          }
        } else {
#pragma unroll
          for (int r = 0; r < FOLD; ++r) {
            const int mm = min(d_row(r, h), M - 1);
            const int p = d[r] - ts[mm * G + g];
            acc[r] += static_cast<float>(p) * sc[u];
          }
        }
      }
    }
  }
  if (PARTIALS) return;

  __syncthreads();
  float* red = reinterpret_cast<float*>(smem);
#pragma unroll
  for (int r = 0; r < FOLD; ++r) red[(wave * FOLD + r) * 64 + lane] = acc[r];
  __syncthreads();
  if (wave == 0) {
    const int nn = n0 + n;
#pragma unroll
    for (int r = 0; r < FOLD; ++r) {
      float v = 0.0f;
#pragma unroll
      for (int w = 0; w < NW; ++w) v += red[(w * FOLD + r) * 64 + lane];
      const int mm = d_row(r, h);
      if (mm < M && nn < N) store_out(y + static_cast<size_t>(mm) * N + nn, v * x_scale[mm]);
    }
  }
}

// ---------------------------------------------------------------- 4-bit GEMV
typedef _Float16 h2 __attribute__((ext_vector_type(2)));

// Eight codes of one packed dword -> the B operand in the order
// [c0, c4, c1, c5, c2, c6, c3, c7] minus the zero point, exactly, as fp16.
__device__ __forceinline__ v8h dequant_w4_f16(uint32_t w, uint32_t neg_magic_z) {
  const h2 nz = __builtin_bit_cast(h2, neg_magic_z);
  h2 r[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    // 0x6400 | c is the fp16 value 1024 + c; adding -(1024 + z) leaves c - z exactly.
    const uint32_t v = ((w >> (4 * s)) & 0x000F000Fu) | 0x64006400u;
    r[s] = __builtin_bit_cast(h2, v) + nz;
  }
  return v8h{r[0].x, r[0].y, r[1].x, r[1].y, r[2].x, r[2].y, r[3].x, r[3].y};
}

// Same for bf16 (no packed bf16 arithmetic on gfx950: via exact fp32 values).
__device__ __forceinline__ v8bf dequant_w4_bf16(uint32_t w, float z) {
  const uint32_t lo = w & 0x0F0F0F0Fu;          // codes 0, 2, 4, 6 in bytes 0..3
  const uint32_t hi = (w >> 4) & 0x0F0F0F0Fu;   // codes 1, 3, 5, 7
  const float c0 = static_cast<float>(lo & 0xFF), c2 = static_cast<float>((lo >> 8) & 0xFF);
  const float c4 = static_cast<float>((lo >> 16) & 0xFF), c6 = static_cast<float>(lo >> 24);
  const float c1 = static_cast<float>(hi & 0xFF), c3 = static_cast<float>((hi >> 8) & 0xFF);
  const float c5 = static_cast<float>((hi >> 16) & 0xFF), c7 = static_cast<float>(hi >> 24);
  return v8bf{static_cast<__bf16>(c0 - z), static_cast<__bf16>(c4 - z),
              static_cast<__bf16>(c1 - z), static_cast<__bf16>(c5 - z),
              static_cast<__bf16>(c2 - z), static_cast<__bf16>(c6 - z),
              static_cast<__bf16>(c3 - z), static_cast<__bf16>(c7 - z)};
}

template <int NW, int FOLD, bool BF, bool ZP, typename TOut>
__global__ __launch_bounds__(NW * 64) void gemv_w4_kernel(
    const uint8_t* __restrict__ codes, const uint16_t* __restrict__ wscale,
    const uint8_t* __restrict__ zeros, const uint16_t* __restrict__ x, int M, int N, int K,
    TOut* __restrict__ y) {
  extern __shared__ __align__(16) uint8_t smem[];
  const int G = K >> 7;
  const int KB = K >> 1;
  const int ZB = (G + 1) >> 1;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n0 = blockIdx.x * kRows;
  uint16_t* xs = reinterpret_cast<uint16_t*>(smem);             // [M][K], 8-chunks permuted

  const int gpw = (G + NW - 1) / NW;
  const int gb = min(G, wave * gpw);
  const int ge = min(G, gb + gpw);
  const int n = lane & 31, h = lane >> 5;
  const int row = min(n0 + n, N - 1);
  const uint8_t* crow = codes + static_cast<size_t>(row) * KB + h * 16;
  const uint16_t* srow = wscale + static_cast<size_t>(row) * G;
  const uint8_t* zrow = ZP ? zeros + static_cast<size_t>(row) * ZB : nullptr;

  constexpr int MG = kMaxG / 2;                // two 16-byte loads per group
  uint4 cw[MG][2];
  float sc[MG];
  int zc[MG];
  auto load_group = [&](int u, int g) {
    cw[u][0] = *reinterpret_cast<const uint4*>(crow + static_cast<size_t>(g) * 64);
    cw[u][1] = *reinterpret_cast<const uint4*>(crow + static_cast<size_t>(g) * 64 + 32);
    const uint16_t sb = srow[g];
    sc[u] = BF ? bf16_to_f32(sb) : __half2float(__builtin_bit_cast(__half, sb));
    zc[u] = ZP ? ((zrow[g >> 1] >> (4 * (g & 1))) & 15) : 8;
  };
#pragma unroll
  for (int u = 0; u < MG; ++u)
    if (gb + u < ge) load_group(u, gb + u);

  // Stage activations: each 8-element chunk stored as [0,4,1,5,2,6,3,7].
  const int chunks = M * (K >> 3);
  for (int c = tid; c < chunks; c += NW * 64) {
    const uint4 v = reinterpret_cast<const uint4*>(x)[c];
    uint4 o;
    o.x = perm_b32(v.z, v.x, 0x05040100u);
    o.y = perm_b32(v.z, v.x, 0x07060302u);
    o.z = perm_b32(v.w, v.y, 0x05040100u);
    o.w = perm_b32(v.w, v.y, 0x07060302u);
    reinterpret_cast<uint4*>(xs)[c] = o;
  }
  __syncthreads();

  const int mA = min(n, M - 1);
  const uint16_t* xa = xs + static_cast<size_t>(mA) * K + h * 32;
  float acc[FOLD];
#pragma unroll
  for (int r = 0; r < FOLD; ++r) acc[r] = 0.0f;

  for (int g0 = gb; g0 < ge; g0 += MG) {
    if (g0 != gb) {
#pragma unroll
      for (int u = 0; u < MG; ++u)
        if (g0 + u < ge) load_group(u, g0 + u);
    }
#pragma unroll
    for (int u = 0; u < MG; ++u) {
      const int g = g0 + u;
      if (g < ge) {
        v16f d = {};
        const uint32_t mz = 0xE400u | static_cast<uint32_t>(zc[u]);   // fp16 -(1024 + z)
        const uint32_t nmz = mz | (mz << 16);
        const float zf = static_cast<float>(zc[u]);
#pragma unroll
        for (int L = 0; L < 2; ++L) {
          const uint32_t wv[4] = {cw[u][L].x, cw[u][L].y, cw[u][L].z, cw[u][L].w};
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            const uint4 araw = *reinterpret_cast<const uint4*>(xa + g * 128 + 64 * L + 8 * s);
            if (BF) {
              const v8bf a = __builtin_bit_cast(v8bf, araw);
              const v8bf b = dequant_w4_bf16(wv[s], zf);
              d = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, d, 0, 0, 0);
            } else {
              const v8h a = __builtin_bit_cast(v8h, araw);
              const v8h b = dequant_w4_f16(wv[s], nmz);
              d = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, d, 0, 0, 0);
            }
          }
        }
#pragma unroll
        for (int r = 0; r < FOLD; ++r) acc[r] = fmaf(sc[u], d[r], acc[r]);
      }
    }
  }

  __syncthreads();
  float* red = reinterpret_cast<float*>(smem);
#pragma unroll
  for (int r = 0; r < FOLD; ++r) red[(wave * FOLD + r) * 64 + lane] = acc[r];
  __syncthreads();
  if (wave == 0) {
    const int nn = n0 + n;
#pragma unroll
    for (int r = 0; r < FOLD; ++r) {
      float v = 0.0f;
#pragma unroll
      for (int w = 0; w < NW; ++w) v += red[(w * FOLD + r) * 64 + lane];
      const int mm = d_row(r, h);
      if (mm < M && nn < N) store_out(y + static_cast<size_t>(mm) * N + nn, v);
    }
  }
}

int fold_for(int64_t m) { return m <= 1 ? 1 : (m <= 8 ? 4 : (m <= 16 ? 8 : 16)); }
int waves_for(int64_t groups) { return groups >= 16 ? 8 : 4; }

template <int NW, int FOLD, typename TOut>
hipError_t t2_go(const bpw_weights& w, const int8_t* q, const float* xs, int m, TOut* y,
                 hipStream_t s) {
  const int n = static_cast<int>(w.n), k = static_cast<int>(w.k), g = k / 128;
  const size_t stage = static_cast<size_t>(m) * k + 4ull * m * g;
  const size_t red = static_cast<size_t>(NW) * FOLD * 64 * 4;
  const size_t lds = stage > red ? stage : red;
  dim3 grid((n + kRows - 1) / kRows), block(NW * 64);
  gemv_t2_kernel<NW, FOLD, TOut, false><<<grid, block, lds, s>>>(
      static_cast<const uint8_t*>(w.codes), static_cast<const __half*>(w.scales), q, xs, m, n, k,
      y, nullptr, 0, 0, 0, 0, 0);
  return hipGetLastError();
}

template <typename TOut>
hipError_t t2_dispatch(const bpw_weights& w, const int8_t* q, const float* xs, int m, TOut* y,
                       hipStream_t s) {
  const int nw = waves_for(w.k / 128);
  const int fold = fold_for(m);
#define BPW_T2(NW_, F_) \
  if (nw == NW_ && fold == F_) return t2_go<NW_, F_, TOut>(w, q, xs, m, y, s);
  BPW_T2(8, 1) BPW_T2(8, 4) BPW_T2(8, 8) BPW_T2(8, 16)
  BPW_T2(4, 1) BPW_T2(4, 4) BPW_T2(4, 8) BPW_T2(4, 16)
#undef BPW_T2
  return hipErrorInvalidValue;
}

template <int NW, int FOLD, bool BF, bool ZP, typename TOut>
hipError_t w4_go(const bpw_weights& w, const uint16_t* x, int m, TOut* y, hipStream_t s) {
  const int n = static_cast<int>(w.n), k = static_cast<int>(w.k);
  const size_t stage = static_cast<size_t>(m) * k * 2;
  const size_t red = static_cast<size_t>(NW) * FOLD * 64 * 4;
  const size_t lds = stage > red ? stage : red;
  dim3 grid((n + kRows - 1) / kRows), block(NW * 64);
  gemv_w4_kernel<NW, FOLD, BF, ZP, TOut><<<grid, block, lds, s>>>(
      static_cast<const uint8_t*>(w.codes), static_cast<const uint16_t*>(w.scales),
      static_cast<const uint8_t*>(w.zeros), x, m, n, k, y);
  return hipGetLastError();
}

template <bool BF, bool ZP, typename TOut>
hipError_t w4_dispatch_f(const bpw_weights& w, const uint16_t* x, int m, TOut* y, hipStream_t s) {
  const int nw = waves_for(w.k / 128);
  const int fold = fold_for(m);
#define BPW_W4(NW_, F_) \
  if (nw == NW_ && fold == F_) return w4_go<NW_, F_, BF, ZP, TOut>(w, x, m, y, s);
  BPW_W4(8, 1) BPW_W4(8, 4) BPW_W4(8, 8) BPW_W4(8, 16)
  BPW_W4(4, 1) BPW_W4(4, 4) BPW_W4(4, 8) BPW_W4(4, 16)
#undef BPW_W4
  return hipErrorInvalidValue;
}

template <typename TOut>
hipError_t w4_dispatch(const bpw_weights& w, const uint16_t* x, bool bf, int m, TOut* y,
                       hipStream_t s) {
  const bool zp = w.fmt == BPW_INT4_ZP;
  if (bf) return zp ? w4_dispatch_f<true, true>(w, x, m, y, s) : w4_dispatch_f<true, false>(w, x, m, y, s);
  return zp ? w4_dispatch_f<false, true>(w, x, m, y, s) : w4_dispatch_f<false, false>(w, x, m, y, s);
}

}  // namespace

bool gemv_t2_fits(int64_t m, int64_t k) {
  return m >= 1 && m <= 32 && static_cast<size_t>(m) * k + 4ull * m * (k / 128) <= kLdsBudget;
}

bool gemv_w4_fits(int64_t m, int64_t k) {
  return m >= 1 && m <= 32 && static_cast<size_t>(m) * k * 2 <= kLdsBudget;
}

hipError_t launch_gemv_t2(const bpw_weights& w, const int8_t* q, const float* x_scale, int64_t m,
                          void* y, int y_dtype, hipStream_t s) {
  const int mi = static_cast<int>(m);
  switch (y_dtype) {
    case BPW_F32: return t2_dispatch(w, q, x_scale, mi, static_cast<float*>(y), s);
    case BPW_F16: return t2_dispatch(w, q, x_scale, mi, static_cast<__half*>(y), s);
    default: return t2_dispatch(w, q, x_scale, mi, static_cast<uint16_t*>(y), s);
  }
}

hipError_t launch_gemv_t2_partials(const bpw_weights& w, const int8_t* q, int64_t m, int64_t m0,
                                   int64_t m1, int64_t n0, int64_t n1, int32_t* out,
                                   hipStream_t s) {
  const int n = static_cast<int>(w.n), k = static_cast<int>(w.k), g = k / 128;
  const int mi = static_cast<int>(m);
  const size_t lds = static_cast<size_t>(mi) * k + 4ull * mi * g;
  const int t0 = static_cast<int>(n0 / kRows), t1 = static_cast<int>((n1 - 1) / kRows);
  dim3 grid(t1 - t0 + 1), block(64 * 8);
  if (waves_for(g) == 8) {
    gemv_t2_kernel<8, 16, float, true><<<grid, block, lds, s>>>(
        static_cast<const uint8_t*>(w.codes), static_cast<const __half*>(w.scales), q, nullptr,
        mi, n, k, nullptr, out, static_cast<int>(m0), static_cast<int>(m1), static_cast<int>(n0),
        static_cast<int>(n1), t0);
  } else {
    block = dim3(64 * 4);
    gemv_t2_kernel<4, 16, float, true><<<grid, block, lds, s>>>(
        static_cast<const uint8_t*>(w.codes), static_cast<const __half*>(w.scales), q, nullptr,
        mi, n, k, nullptr, out, static_cast<int>(m0), static_cast<int>(m1), static_cast<int>(n0),
        static_cast<int>(n1), t0);
  }
  return hipGetLastError();
}

hipError_t launch_gemv_w4(const bpw_weights& w, const void* x_sorted, int x_dtype, int64_t m,
                          void* y, int y_dtype, hipStream_t s) {
  const uint16_t* x = static_cast<const uint16_t*>(x_sorted);
  const bool bf = x_dtype == BPW_BF16;
  const int mi = static_cast<int>(m);
  switch (y_dtype) {
    case BPW_F32: return w4_dispatch(w, x, bf, mi, static_cast<float*>(y), s);
    case BPW_F16: return w4_dispatch(w, x, bf, mi, static_cast<__half*>(y), s);
    default: return w4_dispatch(w, x, bf, mi, static_cast<uint16_t*>(y), s);
  }
}

}  // namespace bpw
