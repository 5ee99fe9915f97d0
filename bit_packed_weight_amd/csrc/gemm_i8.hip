// Ternary weights x int8 activations, prefill-shaped (large M), on gfx950 int8 MFMA.
//
// "Kernel experiments: recorded evidence", Test 7 (INT8 tensor-core MMQ: per
// 128-group an exact integer tile dot, then acc += partial * x_scale * w_scale)
// and Test 21 (code planes of each packed byte multiply plane-ordered
// activations). Here the codes are decoded to signed -1/0/1/2 bytes with one
// byte-select per plane (the table {0xff, 0x00, 0x01, 0x02} of the same page's
// Test 16 decoder), so the int32 MFMA result of a group is the exact partial
// P[m,n,g] and the fold is acc += float(P) * w_scale[n,g]; x_scale[m] is applied
// once at the end.
//
// Workgroup tile 128 (tokens) x 256 (weight rows), 4 waves each 128 x 64; K is
// walked one 128-group per stage through double-buffered LDS. Activations are
// read in plane order (a reorder pass runs first when the caller passes the
// natural order).
#include "device.h"
#include "launch.h"

namespace bpw {
namespace {

constexpr int BM = 128, BN = 256, NT = 256;
constexpr int A_STRIDE = 144;   // 128 bytes + 16 pad: conflict-free 16-byte LDS reads
constexpr int B_STRIDE = 48;    // 32 bytes + 16 pad
constexpr int A_BYTES = BM * A_STRIDE;
constexpr int B_BYTES = BN * B_STRIDE;
constexpr int S_BYTES = BN * 4;
constexpr int STAGE_BYTES = A_BYTES + B_BYTES + S_BYTES;

__device__ __forceinline__ int d_row(int r, int h) { return 8 * (r >> 2) + 4 * h + (r & 3); }

template <typename TOut, bool PARTIALS>
__global__ __launch_bounds__(NT, 1) void gemm_t2_kernel(
    const int8_t* __restrict__ qp, const float* __restrict__ x_scale,
    const uint8_t* __restrict__ codes, const __half* __restrict__ wscale, int M, int N, int K,
    TOut* __restrict__ y, int32_t* __restrict__ pout, int pm0, int pm1, int pn0, int pn1,
    int mt0, int mtiles, int nt0, int ntiles) {
  extern __shared__ __align__(16) uint8_t smem[];
  const int G = K >> 7;
  const int KB = K >> 2;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ntile_all = mtiles * ntiles;
  const int tile = xcd_swizzle(blockIdx.x, ntile_all);
  const int mt = mt0 + tile % mtiles, nt = nt0 + tile / mtiles;
  const int m0 = mt * BM, n0 = nt * BN;

  // Global -> register staging assignments.
  const int8_t* a_src[4];
  int a_dst[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = tid + NT * i;           // 1024 chunks of 16 bytes
    const int r = c >> 3, col = c & 7;
    a_src[i] = qp + static_cast<size_t>(min(m0 + r, M - 1)) * K + col * 16;
    a_dst[i] = r * A_STRIDE + col * 16;
  }
  const uint8_t* b_src[2];
  int b_dst[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int c = tid + NT * i;           // 512 chunks
    const int r = c >> 1, half = c & 1;
    b_src[i] = codes + static_cast<size_t>(min(n0 + r, N - 1)) * KB + half * 16;
    b_dst[i] = A_BYTES + r * B_STRIDE + half * 16;
  }
  const __half* s_src = wscale + static_cast<size_t>(min(n0 + tid, N - 1)) * G;
  const int s_dst = A_BYTES + B_BYTES + tid * 4;

  v4u ra[4], rb[2];
  float rs;
  auto gload = [&](int g) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 4; ++i) ra[i] = *reinterpret_cast<const v4u*>(a_src[i] + g * 128);
#pragma unroll
    for (int i = 0; i < 2; ++i) rb[i] = *reinterpret_cast<const v4u*>(b_src[i] + g * 32);
    rs = __half2float(s_src[g]);
  };
  auto lstore = [&](int buf) __attribute__((always_inline)) {
    uint8_t* base = smem + buf * STAGE_BYTES;
#pragma unroll
    for (int i = 0; i < 4; ++i) *reinterpret_cast<v4u*>(base + a_dst[i]) = ra[i];
#pragma unroll
    for (int i = 0; i < 2; ++i) *reinterpret_cast<v4u*>(base + b_dst[i]) = rb[i];
    *reinterpret_cast<float*>(base + s_dst) = rs;
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

  for (int g = 0; g < G; ++g) {
    const int buf = g & 1;
    if (g + 1 < G) gload(g + 1);
    const uint8_t* base = smem + buf * STAGE_BYTES;
    // B operands of this wave's two 32-row weight tiles, decoded to signed bytes.
    v4i bop[2][4];
    float sj[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int nr = 64 * wave + 32 * j + n;
      const v4u pk = *reinterpret_cast<const v4u*>(base + A_BYTES + nr * B_STRIDE + 16 * h);
#pragma unroll
      for (int t = 0; t < 4; ++t)
        bop[j][t] = v4i{static_cast<int>(code_plane_signed(pk.x, t)),
                        static_cast<int>(code_plane_signed(pk.y, t)),
                        static_cast<int>(code_plane_signed(pk.z, t)),
                        static_cast<int>(code_plane_signed(pk.w, t))};
      sj[j] = *reinterpret_cast<const float*>(base + A_BYTES + B_BYTES + nr * 4);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v4i aop[4];
#pragma unroll
      for (int t = 0; t < 4; ++t)
        aop[t] = *reinterpret_cast<const v4i*>(base + (32 * i + n) * A_STRIDE + 32 * t + 16 * h);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        v16i d = {};
#pragma unroll
        for (int t = 0; t < 4; ++t) d = __builtin_amdgcn_mfma_i32_32x32x32_i8(aop[t], bop[j][t], d, 0, 0, 0);
        if (PARTIALS) {
          const int nn = n0 + 64 * wave + 32 * j + n;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int mm = m0 + 32 * i + d_row(r, h);
            if (mm >= pm0 && mm < pm1 && nn >= pn0 && nn < pn1)
              pout[(static_cast<size_t>(mm - pm0) * (pn1 - pn0) + (nn - pn0)) * G + g] = d[r];
          }
        } else {
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[i][j][r] = fmaf(static_cast<float>(d[r]), sj[j], acc[i][j][r]);
        }
      }
    }
    if (g + 1 < G) lstore(buf ^ 1);
    __syncthreads();
  }
  if (PARTIALS) return;

#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int mm = m0 + 32 * i + d_row(r, h);
      if (mm < M) {
        const float xs = x_scale[mm];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int nn = n0 + 64 * wave + 32 * j + n;
          if (nn < N) store_out(y + static_cast<size_t>(mm) * N + nn, acc[i][j][r] * xs);
        }
      }
    }
  }
}

template <typename TOut>
hipError_t go(const bpw_weights& w, const int8_t* qp, const float* xs, int m, TOut* y,
              hipStream_t s) {
  const int n = static_cast<int>(w.n), k = static_cast<int>(w.k);
  const int mtiles = (m + BM - 1) / BM, ntiles = (n + BN - 1) / BN;
  gemm_t2_kernel<TOut, false><<<mtiles * ntiles, NT, 2 * STAGE_BYTES, s>>>(
      qp, xs, static_cast<const uint8_t*>(w.codes), static_cast<const __half*>(w.scales), m, n, k,
      y, nullptr, 0, 0, 0, 0, 0, mtiles, 0, ntiles);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_t2(const bpw_weights& w, const int8_t* q_planes, const float* x_scale,
                          int64_t m, void* y, int y_dtype, hipStream_t s) {
  const int mi = static_cast<int>(m);
  switch (y_dtype) {
    case BPW_F32: return go(w, q_planes, x_scale, mi, static_cast<float*>(y), s);
    case BPW_F16: return go(w, q_planes, x_scale, mi, static_cast<__half*>(y), s);
    default: return go(w, q_planes, x_scale, mi, static_cast<uint16_t*>(y), s);
  }
}

hipError_t launch_gemm_t2_partials(const bpw_weights& w, const int8_t* q_planes, int64_t m,
                                   int64_t m0, int64_t m1, int64_t n0, int64_t n1, int32_t* out,
                                   hipStream_t s) {
  const int n = static_cast<int>(w.n), k = static_cast<int>(w.k);
  const int mt0 = static_cast<int>(m0 / BM), mt1 = static_cast<int>((m1 - 1) / BM);
  const int nt0 = static_cast<int>(n0 / BN), nt1 = static_cast<int>((n1 - 1) / BN);
  const int mtiles = mt1 - mt0 + 1, ntiles = nt1 - nt0 + 1;
  gemm_t2_kernel<float, true><<<mtiles * ntiles, NT, 2 * STAGE_BYTES, s>>>(
      q_planes, nullptr, static_cast<const uint8_t*>(w.codes),
      static_cast<const __half*>(w.scales), static_cast<int>(m), n, k, nullptr, out,
      static_cast<int>(m0), static_cast<int>(m1), static_cast<int>(n0), static_cast<int>(n1),
      mt0, mtiles, nt0, ntiles);
  return hipGetLastError();
}

}  // namespace bpw
