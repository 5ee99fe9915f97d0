// 4-bit weights x fp16/bf16 activations, prefill-shaped (large M), on gfx950 MFMA.
//
// "mate: Marlin-class W4A16 GEMM for mp_31 (SQMMA int4 x fp16) - #6": the
// prefill kernel unpacks int4 to the activation type before the matrix
// instruction. Each weight is dequantised once per workgroup to
// round-to-nearest-even of (code - zero) * scale in the activation dtype (exact
// in fp32 before that single rounding) and fed to fp16/bf16 MFMA (32x32x16)
// with fp32 accumulation.
//
// Workgroup tile 256 (tokens) x 256 (weight rows), 4 waves; wave w owns weight
// rows [64w, 64w + 64) of the tile and all 256 tokens (8 x 2 MFMA tiles, the
// accumulators live in AGPRs). The activation tile goes through double-buffered
// LDS (64 columns per stage); each wave dequantises its own weight rows straight
// into B-operand registers, so no weight byte touches LDS and no weight is
// dequantised twice. Within a 64-column stage, lane half h of MFMA step s holds
// columns 32h + 8s .. 32h + 8s + 7 (any column order works as long as A and B
// agree); then one 16-byte code load per lane and weight tile feeds all four
// steps.
#include "device.h"
#include "launch.h"

namespace bpw {
namespace {

constexpr int BM = 256, BN = 256, BK = 64, NT = 256;
constexpr int A_STRIDE = BK * 2 + 16;           // 144 bytes: conflict-free 16-byte LDS reads
constexpr int A_BYTES = BM * A_STRIDE;          // one stage
constexpr int LDS_BYTES = 2 * A_BYTES;

__device__ __forceinline__ int d_row(int r, int h) { return 8 * (r >> 2) + 4 * h + (r & 3); }

typedef float v2f __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));

// Eight codes of one packed dword (byte b: code 2b in the low nibble, 2b+1 in
// the high nibble) -> eight 16-bit weights in that order, each the
// round-to-nearest-even of (code - zero) * scale. A byte select builds the fp32
// value 128 + code (bits 0x43 0c 00 00); one fma with nzs = -(128 + zero) * scale
// gives (code - zero) * scale exactly (all products fit fp32), then a packed
// convert rounds two values at once.
template <bool BF>
__device__ __forceinline__ v4u dequant8(uint32_t w, float s, float nzs) {
  const uint32_t lo = w & 0x0F0F0F0Fu, hi = (w >> 4) & 0x0F0F0F0Fu;
  uint32_t o[4];
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const uint32_t sel = 0x07000C0Cu | (static_cast<uint32_t>(b) << 16);
    const float vl = fmaf(__uint_as_float(perm_b32(0x43000000u, lo, sel)), s, nzs);
    const float vh = fmaf(__uint_as_float(perm_b32(0x43000000u, hi, sel)), s, nzs);
    if (BF)
      o[b] = __builtin_bit_cast(uint32_t, __builtin_convertvector(v2f{vl, vh}, v2bf));
    else
      o[b] = __builtin_bit_cast(uint32_t, __builtin_convertvector(v2f{vl, vh}, v2h));
  }
  return v4u{o[0], o[1], o[2], o[3]};
}

template <bool BF, bool ZP, typename TOut>
__global__ __launch_bounds__(NT, 1) void gemm_w4_kernel(
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
  const int n = lane & 31, h = lane >> 5;

  // A: 256 rows x 128 bytes per stage = 2048 chunks, eight per thread.
  const uint16_t* a_src[8];
  int a_dst[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int c = tid + NT * i;
    const int r = c >> 3, col = c & 7;
    a_src[i] = x + static_cast<size_t>(min(m0 + r, M - 1)) * K + col * 8;
    a_dst[i] = r * A_STRIDE + col * 16;
  }
  // B: this lane's two weight rows (one per 32-row tile of the wave).
  const uint8_t* b_src[2];
  const uint16_t* s_src[2];
  const uint8_t* z_src[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const size_t row = static_cast<size_t>(min(n0 + 64 * wave + 32 * j + n, N - 1));
    b_src[j] = codes + row * KB + 16 * h;
    s_src[j] = wscale + row * G;
    z_src[j] = ZP ? zeros + row * ZB : nullptr;
  }

  v4u ra[8];
  auto a_load = [&](int st) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 8; ++i) ra[i] = *reinterpret_cast<const v4u*>(a_src[i] + st * BK);
  };
  auto a_store = [&](int buf) __attribute__((always_inline)) {
    uint8_t* base = smem + buf * A_BYTES;
#pragma unroll
    for (int i = 0; i < 8; ++i) *reinterpret_cast<v4u*>(base + a_dst[i]) = ra[i];
  };
  // Raw weights of one stage: two 16-byte code loads, their scales and the
  // folded zero term, double-buffered so a load never waits for a dequant.
  struct BRaw {
    v4u c[2];
    float s[2], nz[2];
  };
  auto b_load = [&](BRaw& r, int st) __attribute__((always_inline)) {
    const int g = (st * BK) >> 7;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      r.c[j] = *reinterpret_cast<const v4u*>(b_src[j] + st * (BK / 2));
      const uint16_t sb = s_src[j][g];
      r.s[j] = BF ? bf16_to_f32(sb) : __half2float(__builtin_bit_cast(__half, sb));
      const int z = ZP ? ((z_src[j][g >> 1] >> (4 * (g & 1))) & 15) : 8;
      r.nz[j] = -static_cast<float>(128 + z) * r.s[j];   // exact: 8-bit integer times a 16-bit float
    }
  };
  auto b_dequant_step = [&](const BRaw& r, v4u (&bop)[2][4], int ks) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const uint32_t w = ks == 0 ? r.c[j].x : ks == 1 ? r.c[j].y : ks == 2 ? r.c[j].z : r.c[j].w;
      bop[j][ks] = dequant8<BF>(w, r.s[j], r.nz[j]);
    }
  };

  v16f acc[8][2];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = v16f{};

  // One stage (64 columns): global loads for later stages first; then four
  // MFMA steps over the A tile in LDS buffer `buf` with weights `cur`, each
  // interleaved with a quarter of the dequantisation of the next stage's
  // weights (`raw` -> `nxt`); then the next A tile goes to the other buffer.
  // Scheduling fences keep the loads at the start and the LDS stores at the
  // end, so no wait for a fresh load lands among the MFMAs.
  auto stage = [&](int st, int buf, v4u (&cur)[2][4], v4u (&nxt)[2][4], const BRaw& raw,
                   BRaw& load_into) __attribute__((always_inline)) {
    a_load(min(st + 1, S - 1));
    b_load(load_into, min(st + 2, S - 1));
    __builtin_amdgcn_sched_barrier(0);
    const uint8_t* base = smem + buf * A_BYTES + 64 * h;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      v4u aop[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) aop[i] = *reinterpret_cast<const v4u*>(base + (32 * i + n) * A_STRIDE + 16 * ks);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          if (BF)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, aop[i]),
                                                                __builtin_bit_cast(v8bf, cur[j][ks]), acc[i][j], 0, 0, 0);
          else
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(v8h, aop[i]),
                                                               __builtin_bit_cast(v8h, cur[j][ks]), acc[i][j], 0, 0, 0);
        }
      }
      b_dequant_step(raw, nxt, ks);
      // 8 LDS reads, then 16 x (1 MFMA + 3 VALU).
      __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    a_store(buf ^ 1);
  };

  v4u bop0[2][4], bop1[2][4];
  BRaw raw0, raw1;
  a_load(0);
  b_load(raw0, 0);
  a_store(0);
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) b_dequant_step(raw0, bop0, ks);
  b_load(raw0, min(1, S - 1));
  __syncthreads();

  for (int st = 0; st < S; st += 2) {     // S = K / 64 is even
    stage(st, 0, bop0, bop1, raw0, raw1);       // dequant stage st+1 from raw0, load st+2 into raw1
    __syncthreads();
    stage(st + 1, 1, bop1, bop0, raw1, raw0);   // dequant stage st+2 from raw1, load st+3 into raw0
    __syncthreads();
  }

#pragma unroll
  for (int i = 0; i < 8; ++i) {
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
  allow_lds(gemm_w4_kernel<BF, ZP, TOut>, LDS_BYTES);
  gemm_w4_kernel<BF, ZP, TOut><<<mtiles * ntiles, NT, LDS_BYTES, s>>>(
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
