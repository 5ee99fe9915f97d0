// 4-bit weights x fp16/bf16 activations, prefill-shaped (large M), on gfx950 MFMA.
//
// "mate: Marlin-class W4A16 GEMM for mp_31 (SQMMA int4 x fp16) - #6": the
// prefill kernel unpacks int4 to the activation type before the matrix
// instruction. Each workgroup stage dequantises its weight tile once into LDS as
// round-to-nearest-even of (code - zero) * scale in the activation dtype (the
// product is exact in fp32 before that single rounding), then all waves feed
// fp16/bf16 MFMA (32x32x16) with fp32 accumulation.
//
// Workgroup tile 128 (tokens) x 256 (weight rows), 4 waves each 128 x 64; K is
// walked 32 columns per stage through double-buffered LDS.
#include "device.h"
#include "launch.h"

namespace bpw {
namespace {

constexpr int BM = 128, BN = 256, BK = 32, NT = 256;
constexpr int ROW_STRIDE = BK * 2 + 16;         // 80 bytes: conflict-free 16-byte reads
constexpr int A_BYTES = BM * ROW_STRIDE;
constexpr int B_BYTES = BN * ROW_STRIDE;
constexpr int STAGE_BYTES = A_BYTES + B_BYTES;

__device__ __forceinline__ int d_row(int r, int h) { return 8 * (r >> 2) + 4 * h + (r & 3); }

__device__ __forceinline__ uint32_t pack2(float a, float b, bool bf) {
  if (bf) {
    const __bf16 x = static_cast<__bf16>(a), y = static_cast<__bf16>(b);
    return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, x)) |
           (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, y)) << 16);
  }
  const __half x = __float2half_rn(a), y = __float2half_rn(b);
  return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, x)) |
         (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, y)) << 16);
}

template <bool BF, bool ZP, typename TOut>
__global__ __launch_bounds__(NT, 2) void gemm_w4_kernel(
    const uint16_t* __restrict__ x, const uint8_t* __restrict__ codes,
    const uint16_t* __restrict__ wscale, const uint8_t* __restrict__ zeros, int M, int N, int K,
    TOut* __restrict__ y, int mtiles, int ntiles) {
  extern __shared__ __align__(16) uint8_t smem[];
  const int G = K >> 7;
  const int KB = K >> 1;
  const int ZB = (G + 1) >> 1;
  const int S = K / BK;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int tile = xcd_swizzle(blockIdx.x, mtiles * ntiles);
  const int mt = tile % mtiles, nt = tile / mtiles;
  const int m0 = mt * BM, n0 = nt * BN;

  // A: 128 rows x 64 bytes per stage = 512 chunks, two per thread.
  const uint16_t* a_src[2];
  int a_dst[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int c = tid + NT * i;
    const int r = c >> 2, col = c & 3;
    a_src[i] = x + static_cast<size_t>(min(m0 + r, M - 1)) * K + col * 8;
    a_dst[i] = r * ROW_STRIDE + col * 16;
  }
  // B: one weight row per thread, 16 packed bytes (32 codes) per stage.
  const int brow = min(n0 + tid, N - 1);
  const uint8_t* b_src = codes + static_cast<size_t>(brow) * KB;
  const uint16_t* s_src = wscale + static_cast<size_t>(brow) * G;
  const uint8_t* z_src = ZP ? zeros + static_cast<size_t>(brow) * ZB : nullptr;
  const int b_dst = A_BYTES + tid * ROW_STRIDE;

  uint4 ra[2], rb;
  float rsc, rzs;
  auto gload = [&](int st) {
    const int k0 = st * BK;
#pragma unroll
    for (int i = 0; i < 2; ++i) ra[i] = *reinterpret_cast<const uint4*>(a_src[i] + k0);
    rb = *reinterpret_cast<const uint4*>(b_src + k0 / 2);
    const int g = k0 >> 7;
    const uint16_t sb = s_src[g];
    rsc = BF ? bf16_to_f32(sb) : __half2float(__builtin_bit_cast(__half, sb));
    const int z = ZP ? ((z_src[g >> 1] >> (4 * (g & 1))) & 15) : 8;
    rzs = static_cast<float>(z) * rsc;     // exact: small integer times a 16-bit float
  };
  auto lstore = [&](int buf) {
    uint8_t* base = smem + buf * STAGE_BYTES;
#pragma unroll
    for (int i = 0; i < 2; ++i) *reinterpret_cast<uint4*>(base + a_dst[i]) = ra[i];
    // Dequantise 32 codes: (c - z) * s = fma(c, s, -z*s), exact, then one rounding.
    const uint32_t wv[4] = {rb.x, rb.y, rb.z, rb.w};
    uint32_t o[16];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const uint32_t byte = (wv[d] >> (8 * b)) & 0xFFu;
        const float lo = fmaf(static_cast<float>(byte & 15u), rsc, -rzs);
        const float hi = fmaf(static_cast<float>(byte >> 4), rsc, -rzs);
        o[4 * d + b] = pack2(lo, hi, BF);
      }
    }
    uint4* dst = reinterpret_cast<uint4*>(base + b_dst);
#pragma unroll
    for (int i = 0; i < 4; ++i) dst[i] = make_uint4(o[4 * i], o[4 * i + 1], o[4 * i + 2], o[4 * i + 3]);
  };

  const int n = lane & 31, h = lane >> 5;
  v16f acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = v16f{};

  gload(0);
  lstore(0);
  __syncthreads();

  for (int st = 0; st < S; ++st) {
    const int buf = st & 1;
    if (st + 1 < S) gload(st + 1);
    const uint8_t* base = smem + buf * STAGE_BYTES;
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      uint4 bop[2];
#pragma unroll
      for (int j = 0; j < 2; ++j)
        bop[j] = *reinterpret_cast<const uint4*>(base + A_BYTES + (64 * wave + 32 * j + n) * ROW_STRIDE + 32 * ks + 16 * h);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint4 aop = *reinterpret_cast<const uint4*>(base + (32 * i + n) * ROW_STRIDE + 32 * ks + 16 * h);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          if (BF)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, aop),
                                                                __builtin_bit_cast(v8bf, bop[j]), acc[i][j], 0, 0, 0);
          else
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(v8h, aop),
                                                               __builtin_bit_cast(v8h, bop[j]), acc[i][j], 0, 0, 0);
        }
      }
    }
    if (st + 1 < S) lstore(buf ^ 1);
    __syncthreads();
  }

#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int mm = m0 + 32 * i + d_row(r, h);
      if (mm < M) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int nn = n0 + 64 * wave + 32 * j + n;
          if (nn < N) store_out(y + static_cast<size_t>(mm) * N + nn, acc[i][j][r]);
        }
      }
    }
  }
}

template <bool BF, bool ZP, typename TOut>
hipError_t go(const bpw_weights& w, const uint16_t* x, int m, TOut* y, hipStream_t s) {
  const int n = static_cast<int>(w.n), k = static_cast<int>(w.k);
  const int mtiles = (m + BM - 1) / BM, ntiles = (n + BN - 1) / BN;
  gemm_w4_kernel<BF, ZP, TOut><<<mtiles * ntiles, NT, 2 * STAGE_BYTES, s>>>(
      x, static_cast<const uint8_t*>(w.codes), static_cast<const uint16_t*>(w.scales),
      static_cast<const uint8_t*>(w.zeros), m, n, k, y, mtiles, ntiles);
  return hipGetLastError();
}

template <typename TOut>
hipError_t dispatch(const bpw_weights& w, const uint16_t* x, bool bf, int m, TOut* y,
                    hipStream_t s) {
  const bool zp = w.fmt == BPW_INT4_ZP;
  if (bf) return zp ? go<true, true>(w, x, m, y, s) : go<true, false>(w, x, m, y, s);
  return zp ? go<false, true>(w, x, m, y, s) : go<false, false>(w, x, m, y, s);
}

}  // namespace

hipError_t launch_gemm_w4(const bpw_weights& w, const void* x_sorted, int x_dtype, int64_t m,
                          void* y, int y_dtype, hipStream_t s) {
  const uint16_t* x = static_cast<const uint16_t*>(x_sorted);
  const bool bf = x_dtype == BPW_BF16;
  const int mi = static_cast<int>(m);
  switch (y_dtype) {
    case BPW_F32: return dispatch(w, x, bf, mi, static_cast<float*>(y), s);
    case BPW_F16: return dispatch(w, x, bf, mi, static_cast<__half*>(y), s);
    default: return dispatch(w, x, bf, mi, static_cast<uint16_t*>(y), s);
  }
}

}  // namespace bpw
