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
#include "lds_dma.h"
#include "launch.h"
#include "store.h"

namespace bpw {
namespace {

constexpr int BM = 256, BN = 256, BK = 64, NT = 256;
constexpr int A_ROW = 256;                      // one 128-column group of a row, bytes
constexpr int A_BYTES = BM * A_ROW;             // one LDS buffer (64 KB)
constexpr int LDS_BYTES = 2 * A_BYTES;

__device__ __forceinline__ int d_row(int r, int h) { return 8 * (r >> 2) + 4 * h + (r & 3); }

typedef float v2f __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));

// Eight codes of one packed dword, given as its low nibbles (lo = w & 0x0f0f0f0f)
// and high nibbles (hi) (byte b: code 2b in the low nibble, 2b+1 in the high) -> eight 16-bit weights in that order, each the
// round-to-nearest-even of (code - zero) * scale. A byte select builds the fp32
// value 128 + code (bits 0x43 0c 00 00); one fma with nzs = -(128 + zero) * scale
// gives (code - zero) * scale exactly (all products fit fp32), then a packed
// convert rounds two values at once.
template <bool BF>
__device__ __forceinline__ v4u dequant8(uint32_t lo, uint32_t hi, float s, float nzs) {
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
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int tile = xcd_swizzle(blockIdx.x, mtiles * ntiles);
  const int mt = tile % mtiles, nt = tile / mtiles;
  const int m0 = mt * BM, n0 = nt * BN;
  const int n = lane & 31, h = lane >> 5;

  // A: one 128-column group per LDS buffer, 256 rows x 256 bytes, 16-byte chunk
  // c of row r stored at chunk r*16 + (c ^ (r & 15)) (XOR swizzle: the MFMA
  // reads of 16 consecutive rows hit 16 different bank groups). Filled by direct
  // global->LDS loads: instruction t of wave w writes chunks (16w + t)*64 + lane,
  // i.e. row 64w + 4t + lane/16, and each lane fetches the global chunk that
  // belongs there.
  const int x_lane_row = 64 * wave + (lane >> 4);
  auto a_load_group = [&](int g, int buf) __attribute__((always_inline)) {
    const uint32_t dst = static_cast<uint32_t>(reinterpret_cast<size_t>(smem)) + buf * A_BYTES + wave * 16 * 1024;
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      const int lrow = x_lane_row + 4 * t;
      const int c = (lane & 15) ^ (lrow & 15);
      const uint16_t* src = x + static_cast<size_t>(min(m0 + lrow, M - 1)) * K + g * 128 + c * 8;
      lds_dma16(src, __builtin_amdgcn_readfirstlane(dst + t * 1024));
    }
  };
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

  // Raw weights of one 128-column group: per 32-row tile j and 64-column half
  // u, 16 code bytes; plus the scale and zero bits of the group. They are
  // loaded two groups ahead, so nothing inside a group waits on a load issued
  // in that group (mixing these loads with the LDS-direct A loads would
  // otherwise force full waits).
  struct GRaw {
    v4u c[2][2];          // [u][j]
    uint32_t sb[2], zb[2];
  };
  auto graw_load = [&](GRaw& r, int g) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
#pragma unroll
      for (int u = 0; u < 2; ++u)
        r.c[u][j] = *reinterpret_cast<const v4u*>(b_src[j] + g * (2 * BK / 2) + u * (BK / 2));
      r.sb[j] = s_src[j][g];
      r.zb[j] = ZP ? (static_cast<uint32_t>(z_src[j][g >> 1]) >> (4 * (g & 1))) : 8u;
    }
  };
  // Per-stage dequant inputs: nibble-separated code words, scale, -(128+z)*s.
  struct BPrep {
    uint32_t lo[2][4], hi[2][4];
    float s[2], nz[2];
  };
  auto b_prep = [&](const GRaw& r, int u, BPrep& p) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const uint32_t w[4] = {r.c[u][j].x, r.c[u][j].y, r.c[u][j].z, r.c[u][j].w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        p.lo[j][q] = w[q] & 0x0F0F0F0Fu;
        p.hi[j][q] = (w[q] >> 4) & 0x0F0F0F0Fu;
      }
      p.s[j] = BF ? bf16_to_f32(static_cast<uint16_t>(r.sb[j]))
                  : __half2float(__builtin_bit_cast(__half, static_cast<uint16_t>(r.sb[j])));
      // exact: an 8-bit integer times a 16-bit float
      p.nz[j] = -static_cast<float>(128 + static_cast<int>(r.zb[j] & 15u)) * p.s[j];
    }
  };
  auto b_dequant_step = [&](const BPrep& p, v4u (&bop)[2][4], int ks) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < 2; ++j) bop[j][ks] = dequant8<BF>(p.lo[j][ks], p.hi[j][ks], p.s[j], p.nz[j]);
  };

  v16f acc[8][2];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = v16f{};

  // One 64-column half (u) of group g in LDS buffer g & 1: four MFMA steps with
  // weights `cur`, each interleaved with the next step's A reads and a quarter
  // of the next stage's dequant (`prep` -> `nxt`). The A operands of a step
  // are read one step ahead into aop[step & 1]; the first half's last step
  // already reads the second half's first step (same buffer), so only the
  // first step of a group, right after the barrier that publishes its
  // buffer, waits for its reads.
  const int nsw = n & 15;
  v4u aop[2][8];
  auto a_read_step = [&](int buf, int u, int ks, v4u (&dst)[8]) __attribute__((always_inline)) {
    const uint8_t* base = smem + buf * A_BYTES + n * A_ROW + 16 * ((8 * u + 4 * h + ks) ^ nsw);
#pragma unroll
    for (int i = 0; i < 8; ++i) dst[i] = *reinterpret_cast<const v4u*>(base + i * 32 * A_ROW);
  };
  auto half_stage = [&](int buf, int u, v4u (&cur)[2][4], v4u (&nxt)[2][4], const BPrep& prep)
      __attribute__((always_inline)) {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      if (ks < 3)
        a_read_step(buf, u, ks + 1, aop[(ks + 1) & 1]);
      else if (u == 0)
        a_read_step(buf, 1, 0, aop[0]);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          if (BF)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, aop[ks & 1][i]),
                                                                __builtin_bit_cast(v8bf, cur[j][ks]), acc[i][j], 0, 0, 0);
          else
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(v8h, aop[ks & 1][i]),
                                                               __builtin_bit_cast(v8h, cur[j][ks]), acc[i][j], 0, 0, 0);
        }
      }
      b_dequant_step(prep, nxt, ks);
      // 16 x (1 MFMA + 2 VALU), with the next step's 8 LDS reads spread in.
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  v4u bop0[2][4], bop1[2][4];
  GRaw r0, r1, r2;
  a_load_group(0, 0);
  graw_load(r0, 0);
  graw_load(r1, min(1, G - 1));
  __builtin_amdgcn_s_waitcnt(0);
  {
    BPrep p0;
    b_prep(r0, 0, p0);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) b_dequant_step(p0, bop0, ks);
  }
  __syncthreads();

  for (int g = 0; g < G; ++g) {
    // The first step's A reads go out first, so that the loads and dequant
    // preparation below cover their latency. The next group streams into the
    // other buffer while this one is used; every register read below was
    // loaded at least one group earlier and waited for at the previous barrier.
    a_read_step(g & 1, 0, 0, aop[0]);
    __builtin_amdgcn_sched_barrier(0);
    graw_load(r2, min(g + 2, G - 1));
    BPrep pa, pb;
    b_prep(r0, 1, pa);                 // second half of this group
    b_prep(r1, 0, pb);                 // first half of the next group
    __builtin_amdgcn_sched_barrier(0);
    a_load_group(min(g + 1, G - 1), (g + 1) & 1);
    __builtin_amdgcn_sched_barrier(0);
    half_stage(g & 1, 0, bop0, bop1, pa);
    half_stage(g & 1, 1, bop1, bop0, pb);
    __builtin_amdgcn_s_waitcnt(0);     // the direct A loads and raw weights have landed
    __syncthreads();
    r0 = r1;
    r1 = r2;
  }

  // Epilogue: each 32 x 64 block of the wave goes through LDS (8 KB per wave;
  // the A buffers are free once every wave is past this barrier) so that the
  // output leaves in row segments of 4 values per lane instead of single
  // 2-byte stores.
  __syncthreads();
  float* stage = reinterpret_cast<float*>(smem + wave * 8192);
  const bool vec = (N & 3) == 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) stage[d_row(r, h) * 64 + 32 * j + n] = acc[i][j][r];
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int row = 4 * q + (lane >> 4), c4 = 4 * (lane & 15);
      const v4u raw4 = *reinterpret_cast<const v4u*>(stage + row * 64 + c4);
      const int mm = m0 + 32 * i + row, nn = n0 + 64 * wave + c4;
      if (mm < M) {
        const float v[4] = {__uint_as_float(raw4.x), __uint_as_float(raw4.y), __uint_as_float(raw4.z),
                            __uint_as_float(raw4.w)};
        TOut* dst = y + static_cast<size_t>(mm) * N + nn;
        if (vec && nn + 3 < N) {
          store_out4(dst, v);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (nn + e < N) store_out(dst + e, v[e]);
        }
      }
    }
    __builtin_amdgcn_wave_barrier();
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
