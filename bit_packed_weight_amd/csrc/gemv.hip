// Decode-shaped products (M <= 32) on gfx950 MFMA.
//
// M = 1: each wave streams whole weight rows (every weight byte read from HBM
// exactly once, with fully coalesced 16-byte / 8-byte loads along the row) and
// reduces the row with DPP. M <= 32: a workgroup owns 32 weight rows, its waves
// split K into contiguous group ranges and feed MFMA; activations are staged
// once into LDS in the order the matrix instruction reads them; the per-wave
// fp32 partials are summed across waves in a fixed order.
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
#include <atomic>
#include <type_traits>

#include "device.h"
#include "launch.h"
#include "lds_dma.h"
#include "qrule.h"

namespace bpw {
namespace {

constexpr int kRows = 32;                    // weight rows per workgroup (MFMA width)
constexpr size_t kLdsBudget = 128 * 1024;    // staged activations per workgroup
constexpr int kMaxG = 8;                     // groups kept in flight per wave

typedef _Float16 h2 __attribute__((ext_vector_type(2)));

// D layout of a 32x32 MFMA: lane l holds column l % 32 and rows
// 8*(r/4) + 4*(l/32) + r%4 for its 16 accumulator registers r.
__device__ __forceinline__ int d_row(int r, int h) { return 8 * (r >> 2) + 4 * h + (r & 3); }

// Sum over the 64 lanes of a wave in a fixed order; every lane gets the total.
__device__ __forceinline__ float wave_sum(float v) {
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x141, 0xF, 0xF, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x140, 0xF, 0xF, false));
  // Every row of 16 lanes now holds its row total; the four totals are read
  // into scalar registers and added in the order (row0 + row1) + (row2 + row3).
  const int vi = __builtin_bit_cast(int, v);
  const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(vi, 0));
  const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(vi, 16));
  const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(vi, 32));
  const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(vi, 48));
  return (r0 + r1) + (r2 + r3);
}

// Weight codes are read once per call: streaming (non-temporal) loads, for
// kernels whose load instructions take whole 128-byte lines. Where a line is
// read in 32-byte pieces by several instructions, a streaming load lets the
// cache drop it after the first piece and the rest is fetched again.
template <typename T>
__device__ __forceinline__ T load_stream(const uint8_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const T*>(p));
}

// ---------------------------------------------------------------- ternary, M = 1
// K up to CH * 4096. Each wave streams R whole rows with one 1 KB load
// instruction per 4096 columns: lane l holds the 64 codes of columns
// 64l..64l+63 of each 4096-column chunk (half a 128-group); in a last, partial
// chunk the lanes past K read clamped (in-bounds) addresses and zero their
// activations, so they count nothing (no branch around any load). The lane's 64
// activation bytes sit in registers in plane order; each code plane of a packed
// word is one v_dot4 against the matching activation word; the code - 1 offset
// is minus the half-group sum of q; the half-group partial is folded with its
// fp32 scale and the row total is a wave reduction. GS: x_scale holds one
// scale per 128-group ([K/128]) and joins the weight scale in the fold.
//
// TX = float, __half or uint16_t (bf16 bits): the complete decode call for one
// token, the row quantiser fused in. A workgroup of kFusedWaves waves loads the
// activation row (thread t: the 4 values at 4t + 4 threads i), issues its code rows, takes the
// row max (wave maxima through LDS), quantises its values with the row rule
// into an LDS copy of q and the row scale stays in registers; the waves then
// read their q from LDS. q, the scale and everything after are the same as
// the quantiser launch followed by this kernel on int8 activations, so the
// outputs are the same bits. No early return: every wave meets the barriers.
#ifndef BPW_FUSED_WAVES
#define BPW_FUSED_WAVES 16
#endif
constexpr int kFusedWaves = BPW_FUSED_WAVES;   // waves per workgroup of the fused form

template <int R, int CH, typename TOut, bool PARTIALS, bool GS, typename TX = int8_t>
__global__ __launch_bounds__((std::is_same<TX, int8_t>::value ? 256 : 64 * kFusedWaves)) void gemv_t2_row_kernel(
    const uint8_t* __restrict__ codes, const __half* __restrict__ wscale,
    const TX* __restrict__ q, const float* __restrict__ x_scale, int N, int K,
    TOut* __restrict__ y, int32_t* __restrict__ pout, int pn0, int pn1) {
  constexpr bool FUSED = !std::is_same<TX, int8_t>::value;
  static_assert(!FUSED || (!PARTIALS && !GS), "the fused quantiser serves row-scale products");
  constexpr int NW = FUSED ? kFusedWaves : 4, NJ = FUSED ? CH * 1024 / (64 * NW) : 1;
  __shared__ __align__(16) uint32_t qlds[FUSED ? CH * 1024 : 1];
  __shared__ float wmax[NW];
  const int lane = threadIdx.x & 63, tid = threadIdx.x;
  const int row0 = (blockIdx.x * NW + (threadIdx.x >> 6)) * R;
  if (!FUSED && row0 >= N) return;              // whole wave; without FUSED there are no barriers
  const int KB = K >> 2, G = K >> 7;
  bool ok[CH];                                  // this lane's columns of chunk c lie below K
#pragma unroll
  for (int c = 0; c < CH; ++c) ok[c] = c * 4096 + lane * 64 < K;
  // activations first (small, L2-resident), then the code rows
  v4u qin[CH][4];
  float xf[NJ][4];
  if constexpr (FUSED) {
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int i = 4 * tid + 256 * NW * j;
      if (i < K) {
        ld4(reinterpret_cast<const TX*>(q) + i, xf[j]);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) xf[j][e] = 0.0f;
      }
    }
    // Every wave's activation loads go out before any wave's code loads: the
    // barrier (an execution barrier only; it waits for no load) keeps the
    // L2-resident row from queueing behind the HBM code stream, which the
    // quantiser below waits for (measured on the 4096 x 14336 decode: 7.3 us
    // for the complete call without it, 6.55 with it; 8-wave workgroups 7.3).
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
  } else {
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const v4u* src = reinterpret_cast<const v4u*>(reinterpret_cast<const int8_t*>(q) + min(c * 4096 + lane * 64, K - 64));
#pragma unroll
      for (int i = 0; i < 4; ++i) qin[c][i] = src[i];
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  v4u cw[R][CH];
  float sv[R][CH];
  float xg[CH];                                 // GS: this lane's activation group scale per chunk
#pragma unroll
  for (int c = 0; c < CH; ++c) xg[c] = GS ? x_scale[min(32 * c + (lane >> 1), G - 1)] : 1.0f;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const size_t row = static_cast<size_t>(min(row0 + r, N - 1));
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      cw[r][c] = load_stream<v4u>(codes + row * KB + min(c * 1024 + lane * 16, KB - 16));
      sv[r][c] = __half2float(wscale[row * G + min(32 * c + (lane >> 1), G - 1)]);
    }
  }
  float fused_scale = 0.0f;
  if (FUSED) {
    // the row quantiser's rule, with the code rows in flight (all issued first)
    __builtin_amdgcn_sched_barrier(0);
    float amax = 0.0f, nonfinite = 0.0f;
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        amax = fmaxf(amax, fabsf(xf[j][e]));
        nonfinite = fmaf(xf[j][e], 0.0f, nonfinite);
      }
    if (nonfinite != nonfinite) amax = __builtin_inff();
    amax = wave_max(amax);
    if (lane == 0) wmax[tid >> 6] = amax;
    __syncthreads();
    amax = wmax[0];
#pragma unroll
    for (int v = 1; v < NW; ++v) amax = fmaxf(amax, wmax[v]);
    const bool bad = __builtin_isinf(amax);
    fused_scale = bad ? __builtin_nanf("") : row_scale(amax);
    const float div = fused_scale > 0.0f ? fused_scale : 1.0f;
    // q word w of 64-byte slot l = w / 16 (the 64 bytes one lane reads) goes to
    // 16-byte unit ((w / 4) % 4) ^ (l / 4 % 4) of the slot: the 16 lanes of
    // one 16-byte LDS read then cover all 64 banks (a 4-way conflict
    // unswizzled)
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int i = 4 * tid + 256 * NW * j;
      const int w = i >> 2;
      if (i < K) qlds[(w & ~15) | ((((w >> 2) ^ (w >> 6)) & 3) << 2) | (w & 3)] = bad ? 0u : quantize_word(xf[j], div);
    }
    __syncthreads();
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int l = min(c * 64 + lane, (K >> 6) - 1);
#pragma unroll
      for (int i = 0; i < 4; ++i) qin[c][i] = *reinterpret_cast<const v4u*>(qlds + 16 * l + 4 * (i ^ ((l >> 2) & 3)));
    }
  }
  v4u qp[CH][4];
  int th[CH];
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    v4u in[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) in[i] = ok[c] ? qin[c][i] : v4u{0, 0, 0, 0};
    to_plane_order(in, qp[c]);
    int sum = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sum = sum_i8x4(in[i].x, sum);
      sum = sum_i8x4(in[i].y, sum);
      sum = sum_i8x4(in[i].z, sum);
      sum = sum_i8x4(in[i].w, sum);
    }
    th[c] = sum;
  }
  float acc[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    acc[r] = 0.0f;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const uint32_t wv[4] = {cw[r][c].x, cw[r][c].y, cw[r][c].z, cw[r][c].w};
      const uint32_t qv[4][4] = {{qp[c][0].x, qp[c][0].y, qp[c][0].z, qp[c][0].w},
                                 {qp[c][1].x, qp[c][1].y, qp[c][1].z, qp[c][1].w},
                                 {qp[c][2].x, qp[c][2].y, qp[c][2].z, qp[c][2].w},
                                 {qp[c][3].x, qp[c][3].y, qp[c][3].z, qp[c][3].w}};
      int p = 0;
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int t = 0; t < 4; ++t)
          p = __builtin_amdgcn_sdot4(static_cast<int>(code_plane(wv[u], t)), static_cast<int>(qv[t][u]), p, false);
      p -= th[c];
      if (PARTIALS) {
        const int pg = p + __shfl_xor(p, 1);
        const int row = row0 + r;
        if ((lane & 1) == 0 && ok[c] && row < N && row >= pn0 && row < pn1)
          pout[static_cast<size_t>(row - pn0) * G + 32 * c + (lane >> 1)] = pg;
      } else {
        acc[r] = fmaf(static_cast<float>(p), GS ? sv[r][c] * xg[c] : sv[r][c], acc[r]);
      }
    }
  }
  if (PARTIALS) return;
  const float xs = FUSED ? fused_scale : (GS ? 1.0f : x_scale[0]);
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const float v = wave_sum(acc[r]);
    if (lane == r && row0 + r < N) store_out(y + row0 + r, v * xs);
  }
}

// ---------------------------------------------------------------- ternary, M <= 32, K <= 4096
// Skinny products stream the weights like the M = 1 kernel but feed int8 MFMA.
// One workgroup per CU owns a contiguous slice of weight rows (processed as
// tiles of 32 rows); its NW waves split K, GPW groups each. A wave keeps the
// A operands of its K slice (activations in plane order, all M rows) in
// registers, loaded once, and streams its slice of each weight row straight
// from HBM into B operands: lane (n, h) reads 16 bytes of row n per group, and
// the two lanes of a row together cover its 32-byte group, so the wave reads
// whole 128-byte lines. Codes are decoded signed (the {0xff, 0x00, 0x01, 0x02}
// byte table), so each chain of four MFMAs is the exact partial P[m,n,g]. The
// per-wave fp32 results of a tile are summed in a fixed order through LDS.
//
// SPLIT (split-K for long K): blockIdx.y selects the K slice of NW * GPW groups
// starting at group blockIdx.y * NW * GPW; the workgroup's fixed-order sum over
// its waves goes, unscaled, to part[blockIdx.y][M][N] (fp32), and
// splitk_reduce_kernel adds the slices in slice order and applies x_scale.
template <int NW, int GPW, int MAXT, int FR, typename TOut, bool PARTIALS, bool GS, bool SPLIT = false>
__global__ __launch_bounds__(NW * 64) void gemv_t2_skinny_kernel(
    const uint8_t* __restrict__ codes, const __half* __restrict__ wscale,
    const int8_t* __restrict__ q, const float* __restrict__ x_scale, int M, int N, int K, int rpw,
    TOut* __restrict__ y, int32_t* __restrict__ pout, int pm0, int pm1, int pn0, int pn1, int wg0,
    float* __restrict__ part) {
  // FR: accumulator registers that can hold a token row < M (registers 0..7
  // hold rows 0..15, so 8 when M <= 16, else 16). GS: x_scale holds one scale
  // per (row, 128-group), [M][K/128], and joins the weight scale in the fold.
  extern __shared__ float red[];                           // [tile of a pair][wave][reg][lane]
  const int G = K >> 7, KB = K >> 2;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 31, h = lane >> 5;
  const int r0 = (blockIdx.x + wg0) * rpw;
  const int r1 = min(r0 + rpw, N);
  const int gb = (SPLIT ? blockIdx.y * NW * GPW : 0) + wave * GPW;

  // Loads in the order they are consumed (the hardware counts them in issue
  // order): activations, group scales and row scales first (small, mostly L2
  // hits), then the code stream, tile by tile, group by group.
  // (token rows n >= M are zero in A: their outputs are never stored)
  v4u ain[GPW][4];
#pragma unroll
  for (int u = 0; u < GPW; ++u)
#pragma unroll
    for (int i = 0; i < 4; ++i) ain[u][i] = v4u{0, 0, 0, 0};
  if (n < M) {
#pragma unroll
    for (int u = 0; u < GPW; ++u) {
      const int g = min(gb + u, G - 1);
      const v4u* src = reinterpret_cast<const v4u*>(q + static_cast<size_t>(n) * K + g * 128 + 64 * h);
#pragma unroll
      for (int i = 0; i < 4; ++i) ain[u][i] = src[i];
    }
  }
  __half sc[MAXT][GPW];                                    // converted at use, not at load
  const uint8_t* crow[MAXT];
#pragma unroll
  for (int t = 0; t < MAXT; ++t) {
    // rows past this workgroup's share read its last row again (same address
    // across the wave: no extra traffic) and are never stored
    const size_t row = static_cast<size_t>(min(r0 + 32 * t + n, r1 - 1));
    crow[t] = codes + row * KB + 16 * h;
#pragma unroll
    for (int u = 0; u < GPW; ++u) sc[t][u] = wscale[row * G + min(gb + u, G - 1)];
  }
  // GS: the activation group scales of this wave's groups for 32 token rows,
  // [u][m] in the wave's own LDS slice after the reduction area (loaded here,
  // stored once the code loads are out).
  constexpr int XPL = (GPW * 32 + 63) / 64;
  float* xsl = red + 2 * NW * FR * 64 + wave * (GPW * 32);
  float xst[XPL];
  if (GS) {
#pragma unroll
    for (int c = 0; c < XPL; ++c) {
      const int e = min(lane + 64 * c, GPW * 32 - 1), u = e >> 5, m = e & 31;
      xst[c] = x_scale[min(m, M - 1) * G + min(gb + u, G - 1)];
    }
  }
  // Row scales of the outputs this thread stores (the same rows for every tile).
  constexpr int OPT = (2 * FR + NW - 1) / NW;               // outputs per thread per tile pair
  float xsv[OPT];
  if (!PARTIALS && !GS && !SPLIT) {
#pragma unroll
    for (int k = 0; k < OPT; ++k) {
      const int rl = (tid + k * NW * 64) % (FR * 64);
      xsv[k] = x_scale[min(d_row(rl >> 6, (rl & 63) >> 5), M - 1)];
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  v4u cw[MAXT][GPW];
#pragma unroll
  for (int t = 0; t < MAXT; ++t)
#pragma unroll
    for (int u = 0; u < GPW; ++u) {
      cw[t][u] = *reinterpret_cast<const v4u*>(crow[t] + min(gb + u, G - 1) * 32);
      __builtin_amdgcn_sched_barrier(0);
    }
  if (GS) {
#pragma unroll
    for (int c = 0; c < XPL; ++c)
      if (lane + 64 * c < GPW * 32) xsl[lane + 64 * c] = xst[c];
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
  // Keep the transposes below the code loads (an empty asm on their inputs).
#pragma unroll
  for (int u = 0; u < GPW; ++u)
#pragma unroll
    for (int i = 0; i < 4; ++i) asm volatile("" : "+v"(ain[u][i]));
  // A operands: token row m = n (clamped), half h of each group, plane order.
  v4i a[GPW][4];
#pragma unroll
  for (int u = 0; u < GPW; ++u) {
    v4u o[4];
    to_plane_order(ain[u], o);
#pragma unroll
    for (int t = 0; t < 4; ++t) a[u][t] = __builtin_bit_cast(v4i, o[t]);
  }
  // Tiles in pairs: compute both, then one fixed-order reduction through LDS.
  // Every tile is computed (no branch, so every load above stays hoisted);
  // the stores drop rows past the workgroup's share.
#pragma unroll
  for (int t0 = 0; t0 < MAXT; t0 += 2) {
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const int t = t0 + tt;
      float acc[FR];
#pragma unroll
      for (int r = 0; r < FR; ++r) acc[r] = 0.0f;
#pragma unroll
      for (int u = 0; u < GPW; ++u) {
        // Groups past the end (the last wave of a ragged K) run on clamped
        // data and count for nothing: no branch, so the loads stay hoisted.
        const int g = gb + u;
        {
          const v4u c = cw[t][u];
          v16i d = {};
#pragma unroll
          for (int p = 0; p < 4; ++p) {
            const v4i b = {static_cast<int>(code_plane_signed(c.x, p)), static_cast<int>(code_plane_signed(c.y, p)),
                           static_cast<int>(code_plane_signed(c.z, p)), static_cast<int>(code_plane_signed(c.w, p))};
            d = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[u][p], b, d, 0, 0, 0);
          }
          if (PARTIALS) {
            const int nn = r0 + 32 * t + n;
#pragma unroll
            for (int r = 0; r < FR; ++r) {
              const int mm = d_row(r, h);
              if (g < G && mm < M && mm >= pm0 && mm < pm1 && nn < r1 && nn >= pn0 && nn < pn1)
                pout[(static_cast<size_t>(mm - pm0) * (pn1 - pn0) + (nn - pn0)) * G + g] = d[r];
            }
          } else {
            const float sg = g < G ? __half2float(sc[t][u]) : 0.0f;
#pragma unroll
            for (int r = 0; r < FR; ++r)
              acc[r] = fmaf(static_cast<float>(d[r]), GS ? sg * xsl[u * 32 + d_row(r, h)] : sg, acc[r]);
          }
        }
      }
      if (!PARTIALS) {
#pragma unroll
        for (int r = 0; r < FR; ++r) red[((tt * NW + wave) * FR + r) * 64 + lane] = acc[r];
      }
    }
    if (PARTIALS) continue;
    __syncthreads();
#pragma unroll
    for (int k = 0; k < OPT; ++k) {
      // The sum and the scaling run unconditionally (the row-scale load is
      // then not sunk behind the barrier); only the store is guarded.
      const int o0 = tid + k * NW * 64, o = min(o0, 2 * FR * 64 - 1);
      const int tt = o / (FR * 64), rl = o - tt * FR * 64, r = rl >> 6, l = rl & 63;
      float v = 0.0f;
#pragma unroll
      for (int w = 0; w < NW; ++w) v += red[((tt * NW + w) * FR + r) * 64 + l];
      if (!GS && !SPLIT) v *= xsv[k];
      const int mm = d_row(r, l >> 5), nn = r0 + 32 * (t0 + tt) + (l & 31);
      if (SPLIT) {
        if (o0 == o && mm < M && nn < r1) part[(static_cast<size_t>(blockIdx.y) * M + mm) * N + nn] = v;
      } else if (o0 == o && mm < M && nn < r1) {
        store_out(y + static_cast<size_t>(mm) * N + nn, v);
      }
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------- ternary, M <= 16, K <= 4096, staged in LDS
// One workgroup of 16 waves per CU takes rpw <= 64 weight rows (four 16-row
// tiles) over the whole K; wave w owns groups GPW * w .. GPW * w + GPW - 1.
// Every global read is a direct global -> LDS copy issued up front, so the
// code stream leaves HBM in whole contiguous rows (one 1 KB copy per row of
// K = 4096): the wave's activations (16 tokens of its groups), a share of the
// scale block and of the activation scales, then one code row of each tile,
// tile by tile. A tile is computed once every wave's copy of it has landed
// (vmcnt over the copies issued after it, then a barrier), while the later
// tiles stream in. MFMA i32_16x16x64_i8: lane (n, j) = (l % 16, l / 16) holds
// token n of A and weight row n of the tile for B, 16 of the group's columns
// per instruction (two instructions per 128-group). The codes are decoded
// unsigned (each plane is one shift and one mask) and the code - 1 offset
// enters as the MFMA's starting accumulator, -sum(q) over the group per token,
// itself an MFMA of the activations against a B of all -1 ("Kernel
// experiments: recorded evidence", Test 21: minus the group sum of q). The
// per-wave fp32 results meet in LDS, summed in a fixed order.
constexpr int kStageWaves = 16, kStageTiles = 4;

struct T2StageLds {
  int rs, oc, oa, os, ox, red, total;   // code row stride; byte offsets; bytes
};

__host__ __device__ inline T2StageLds t2_stage_lds(int K, int G, int gpw, int xs_bytes) {
  T2StageLds l;
  l.rs = (K >> 2) + 16;
  l.oc = 0;
  const int codes = kStageTiles * 16 * l.rs;
  const int red = kStageTiles * kStageWaves * 4 * 64 * 4;   // fp32 partials, after the codes are read
  l.red = 0;
  l.oa = (codes > red ? codes : red);
  l.os = l.oa + kStageWaves * gpw * 16 * 128;
  l.ox = l.os + ((kStageTiles * 16 * G * 2 + 15) & ~15);
  l.total = l.ox + ((xs_bytes + 15) & ~15);
  return l;
}

// SPLIT: slice blockIdx.y of 32 groups (4096 columns; the last slice what is
// left, a multiple of 1024) per workgroup, its fp32 sums before the activation
// scale written to part[slice][m][n] for splitk_reduce_kernel, which adds the
// slices in slice order and applies x_scale.
template <int GPW, typename TOut, bool PARTIALS, bool GS, bool SPLIT = false>
__global__ __launch_bounds__(64 * kStageWaves) void gemv_t2_stage_kernel(
    const uint8_t* __restrict__ codes, const __half* __restrict__ wscale,
    const int8_t* __restrict__ q, const float* __restrict__ x_scale, int M, int N, int K, int rpw,
    TOut* __restrict__ y, int32_t* __restrict__ pout, int pm0, int pm1, int pn0, int pn1, float* __restrict__ part) {
  constexpr int NW = kStageWaves, T = kStageTiles;
  static_assert(!SPLIT || (!PARTIALS && !GS), "the K-sliced form takes row scales only");
  extern __shared__ __align__(16) uint8_t stg[];
  // G, KB: groups and code bytes per row of this workgroup's K range (the
  // whole K, or one slice); GA, KBA: of the whole row
  const int GA = K >> 7, KBA = K >> 2;
  const int sl = SPLIT ? static_cast<int>(blockIdx.y) : 0;
  const int g0 = 32 * sl;                                   // first group of the slice
  const int G = SPLIT ? min(32, GA - g0) : GA, KB = 32 * G;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, j = lane >> 4;
  const int r0 = blockIdx.x * rpw;
  const int nrow = min(rpw, N - r0);                       // >= 1
  const int gb = wave * GPW;
  const int xs_bytes = (PARTIALS || SPLIT) ? 0 : (GS ? M * G * 4 : M * 4);
  const T2StageLds L = t2_stage_lds(128 * G, G, GPW, xs_bytes);
  const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<size_t>(stg));

  // ---- copies, in the order they are waited for
  // the workgroup's scale block (nrow x G fp16, contiguous; G % 8 == 0 keeps
  // it whole 16-byte pieces) and the activation scales, one piece per wave
  // from wave 0 on: 1 KB pieces, or M floats 4 bytes per lane. (A transposed
  // copy, 4 bytes per lane, reads its scales without bank conflicts but
  // measured slower: 7.23 against 7.06 us at M=16.)
  if (!PARTIALS) {
    const int sb = nrow * G * 2, npieces = (sb + 1023) >> 10;
    const int xpieces = SPLIT ? 0 : GS ? (xs_bytes + 1023) >> 10 : 1;
    if (wave < npieces) {
      const int off = wave * 1024 + lane * 16;
      if (off < sb) {
        // (a slice's rows are G of the row's GA scales: row off / (2G), piece
        // of it (off % (2G)) / 16; 2G is a multiple of 16)
        const size_t src = SPLIT ? (static_cast<size_t>(r0) + off / (2 * G)) * GA * 2 + g0 * 2 + off % (2 * G)
                                 : static_cast<size_t>(r0) * G * 2 + off;
        lds_dma16(reinterpret_cast<const uint8_t*>(wscale) + src,
                  __builtin_amdgcn_readfirstlane(lds0 + L.os + wave * 1024));
      }
    } else if (wave < npieces + xpieces) {
      const int pc = wave - npieces;
      if (GS) {
        const int off = pc * 1024 + lane * 16;           // M * G * 4 bytes, a multiple of 16
        if (off < xs_bytes)
          lds_dma16(reinterpret_cast<const uint8_t*>(x_scale) + off,
                    __builtin_amdgcn_readfirstlane(lds0 + L.ox + pc * 1024));
      } else if (lane < M) {
        lds_dma4(x_scale + lane, __builtin_amdgcn_readfirstlane(lds0 + L.ox));
      }
    }
  }
  // activations of this wave's groups: 16 tokens x 128 bytes per group, two
  // 1 KB copies (tokens past M repeat token M - 1; their outputs are dropped)
#pragma unroll
  for (int u = 0; u < GPW; ++u) {
    const int g = min(gb + u, G - 1);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      // token 8h + l / 8, its 16-byte unit (l % 8) ^ token % 8 lands in slot l % 8:
      // the A reads below, eight tokens at one unit, then fall in distinct banks
      const int tk = 8 * h + (lane >> 3), m = min(tk, M - 1);
      lds_dma16(q + static_cast<size_t>(m) * K + (g0 + g) * 128 + 16 * ((lane & 7) ^ (tk & 7)),
                __builtin_amdgcn_readfirstlane(lds0 + L.oa + ((wave * GPW + u) * 2 + h) * 1024));
    }
  }
  // every wave's scale and activation copies go out before any wave's code
  // rows (an execution barrier; it waits for no copy)
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  // one code row per tile (rows past the workgroup's share repeat its last
  // row): tiles 0 and 1 now, each later one after the tile two before it is
  // computed, so two tiles are in flight (PARTIALS: all four now)
  auto copy_tile = [&](int t) {
    const int row = min(16 * t + wave, nrow - 1);
    if (lane * 16 < KB)
      lds_dma16(codes + static_cast<size_t>(r0 + row) * KBA + 32 * g0 + lane * 16,
                __builtin_amdgcn_readfirstlane(lds0 + L.oc + (16 * t + wave) * L.rs));
  };
  static_assert(T == 4, "the copy schedule and the waits below count four tiles");
  copy_tile(0);
  copy_tile(1);
  if (PARTIALS) {
    copy_tile(2);
    copy_tile(3);
  }

  // ---- this wave's activations have landed (tiles 0 and 1 are in flight)
  // (PARTIALS stores inside the tile loop, and stores count in vmcnt too: that
  // verification path waits for every copy here instead)
  if (PARTIALS) {
    wait_vmcnt<0>();
    __syncthreads();
  } else {
    // (the compiler sees neither the copies nor this wait as LDS traffic:
    // the reads below are pinned after it)
    __builtin_amdgcn_sched_barrier(0);
    wait_vmcnt<2>();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  }
  // A operands: token n, columns 32j + 16e .. + 15 of group u, as the 4x4
  // byte transpose the code planes need (plane p, byte i <-> column 4i + p)
  v4i a[GPW][2], cneg[GPW];
  const v4i neg1 = {-1, -1, -1, -1};
#pragma unroll
  for (int u = 0; u < GPW; ++u) {
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const v4u v = *reinterpret_cast<const v4u*>(stg + L.oa + (wave * GPW + u) * 2048 + n * 128 +
                                                   16 * ((2 * j + e) ^ (n & 7)));
      uint32_t o0, o1, o2, o3;
      transpose4x4(v.x, v.y, v.z, v.w, o0, o1, o2, o3);
      a[u][e] = v4i{static_cast<int>(o0), static_cast<int>(o1), static_cast<int>(o2), static_cast<int>(o3)};
    }
    // -sum(q) of token 4j + r over the group, in every column
    v4i c = {0, 0, 0, 0};
    c = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[u][0], neg1, c, 0, 0, 0);
    cneg[u] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[u][1], neg1, c, 0, 0, 0);
  }
  // ---- tile 0 and every wave's scales have landed
  if (!PARTIALS) {
    wait_vmcnt<1>();
    __syncthreads();
  }
  float acc[T][4];
#pragma unroll
  for (int t = 0; t < T; ++t)
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[t][r] = 0.0f;
#pragma unroll
  for (int t = 0; t < T; ++t) {
    if (t > 0 && !PARTIALS) {
      // the copies of tile t: all but tile t + 1's, if issued
      if (t < T - 1) wait_vmcnt<1>();
      else wait_vmcnt<0>();
      __syncthreads();
    }
    // (after the barrier: every wave is done with tile t - 1's rows; tile
    // t + 2's slots were never read)
    if (!PARTIALS && t + 2 < T) copy_tile(t + 2);
    const uint8_t* crow = stg + L.oc + (16 * t + n) * L.rs;
#pragma unroll
    for (int u = 0; u < GPW; ++u) {
      const int g = gb + u;
      const int gc = min(g, G - 1);
      const v2u w2 = *reinterpret_cast<const v2u*>(crow + gc * 32 + 8 * j);
      v4i d = cneg[u];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const uint32_t w = e ? w2.y : w2.x;
        const v4i b = {static_cast<int>(code_plane(w, 0)), static_cast<int>(code_plane(w, 1)),
                       static_cast<int>(code_plane(w, 2)), static_cast<int>(code_plane(w, 3))};
        d = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[u][e], b, d, 0, 0, 0);
      }
      const int nn = r0 + 16 * t + n;                      // weight row of this lane
      if (PARTIALS) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int mm = 4 * j + r;
          if (g < G && mm < M && mm >= pm0 && mm < pm1 && 16 * t + n < nrow && nn >= pn0 && nn < pn1)
            pout[(static_cast<size_t>(mm - pm0) * (pn1 - pn0) + (nn - pn0)) * G + g] = d[r];
        }
      } else {
        const __half hs = reinterpret_cast<const __half*>(stg + L.os)[min(16 * t + n, nrow - 1) * G + gc];
        const float sg = g < G ? __half2float(hs) : 0.0f;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float xg = GS ? reinterpret_cast<const float*>(stg + L.ox)[min(4 * j + r, M - 1) * G + gc] : 1.0f;
          acc[t][r] = fmaf(static_cast<float>(d[r]), GS ? sg * xg : sg, acc[t][r]);
        }
      }
    }
  }
  if (PARTIALS) return;
  // ---- fixed-order sum over the waves (the code rows are no longer read)
  __syncthreads();
  float* red = reinterpret_cast<float*>(stg + L.red);
#pragma unroll
  for (int t = 0; t < T; ++t)
#pragma unroll
    for (int r = 0; r < 4; ++r) red[((t * NW + wave) * 4 + r) * 64 + lane] = acc[t][r];
  __syncthreads();
  {
    // one output per thread: tile t, register r, lane l
    const int t = tid >> 8, r = (tid >> 6) & 3, l = tid & 63;
    float v = 0.0f;
#pragma unroll
    for (int w = 0; w < NW; ++w) v += red[((t * NW + w) * 4 + r) * 64 + l];
    const int mm = 4 * (l >> 4) + r, rl = 16 * t + (l & 15);
    if (SPLIT) {
      if (mm < M && rl < nrow) part[(static_cast<size_t>(sl) * M + mm) * N + r0 + rl] = v;
    } else {
      if (!GS) v *= reinterpret_cast<const float*>(stg + L.ox)[min(mm, M - 1)];
      if (mm < M && rl < nrow) store_out(y + static_cast<size_t>(mm) * N + r0 + rl, v);
    }
  }
}

// ---------------------------------------------------------------- ternary, M <= 32, long K
// The skinny kernel's scheme for K beyond what one wave's registers hold: the
// waves step through K in phases of NW * 2 groups (2 per wave), loading a
// phase's activations, scales and codes together and accumulating two 32-row
// tiles (rpw <= 64) in fp32 across the phases; one fixed-order reduction
// through LDS at the end.
template <int NW, int FR, typename TOut, bool PARTIALS, bool GS>
__global__ __launch_bounds__(NW * 64) void gemv_t2_long_kernel(
    const uint8_t* __restrict__ codes, const __half* __restrict__ wscale,
    const int8_t* __restrict__ q, const float* __restrict__ x_scale, int M, int N, int K, int rpw,
    TOut* __restrict__ y, int32_t* __restrict__ pout, int pm0, int pm1, int pn0, int pn1, int wg0) {
  constexpr int GPW = 2;
  extern __shared__ float red[];                           // [tile][wave][reg][lane], then GS scales
  const int G = K >> 7, KB = K >> 2;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 31, h = lane >> 5;
  const int r0 = (blockIdx.x + wg0) * rpw;
  const int r1 = min(r0 + rpw, N);
  const int nph = (G + NW * GPW - 1) / (NW * GPW);
  const uint8_t* crow[2];
  const __half* srow[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const size_t row = static_cast<size_t>(min(r0 + 32 * t + n, r1 - 1));
    crow[t] = codes + row * KB + 16 * h;
    srow[t] = wscale + row * G;
  }
  constexpr int OPT = (2 * FR + NW - 1) / NW;
  float xsv[OPT];
  if (!PARTIALS && !GS) {
#pragma unroll
    for (int k = 0; k < OPT; ++k) {
      const int rl = (tid + k * NW * 64) % (FR * 64);
      xsv[k] = x_scale[min(d_row(rl >> 6, (rl & 63) >> 5), M - 1)];
    }
  }
  float* xsl = red + 2 * NW * FR * 64 + wave * (GPW * 32);
  float acc[2][FR];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int r = 0; r < FR; ++r) acc[t][r] = 0.0f;
  for (int ph = 0; ph < nph; ++ph) {
    const int gb = (ph * NW + wave) * GPW;
    v4u ain[GPW][4];
#pragma unroll
    for (int u = 0; u < GPW; ++u)
#pragma unroll
      for (int i = 0; i < 4; ++i) ain[u][i] = v4u{0, 0, 0, 0};
    if (n < M) {
#pragma unroll
      for (int u = 0; u < GPW; ++u) {
        const v4u* src = reinterpret_cast<const v4u*>(q + static_cast<size_t>(n) * K + min(gb + u, G - 1) * 128 + 64 * h);
#pragma unroll
        for (int i = 0; i < 4; ++i) ain[u][i] = src[i];
      }
    }
    __half sc[2][GPW];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int u = 0; u < GPW; ++u) sc[t][u] = srow[t][min(gb + u, G - 1)];
    float xst = 0.0f;                                      // GS: element lane of this wave's [u][m] block
    if (GS) xst = x_scale[min(lane & 31, M - 1) * G + min(gb + (lane >> 5), G - 1)];
    __builtin_amdgcn_sched_barrier(0);
    v4u cw[2][GPW];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int u = 0; u < GPW; ++u) {
        cw[t][u] = *reinterpret_cast<const v4u*>(crow[t] + min(gb + u, G - 1) * 32);
        __builtin_amdgcn_sched_barrier(0);
      }
    if (GS) {
      // the previous phase's reads of the slice are done (their values were used)
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      xsl[lane] = xst;                                     // 64 = GPW * 32 elements
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
    v4i a[GPW][4];
#pragma unroll
    for (int u = 0; u < GPW; ++u) {
      v4u o[4];
      to_plane_order(ain[u], o);
#pragma unroll
      for (int t = 0; t < 4; ++t) a[u][t] = __builtin_bit_cast(v4i, o[t]);
    }
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int u = 0; u < GPW; ++u) {
        const int g = gb + u;                              // past the end: clamped data, zero weight
        const v4u c = cw[t][u];
        v16i d = {};
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const v4i b = {static_cast<int>(code_plane_signed(c.x, p)), static_cast<int>(code_plane_signed(c.y, p)),
                         static_cast<int>(code_plane_signed(c.z, p)), static_cast<int>(code_plane_signed(c.w, p))};
          d = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[u][p], b, d, 0, 0, 0);
        }
        if (PARTIALS) {
          const int nn = r0 + 32 * t + n;
#pragma unroll
          for (int r = 0; r < FR; ++r) {
            const int mm = d_row(r, h);
            if (g < G && mm < M && mm >= pm0 && mm < pm1 && nn < r1 && nn >= pn0 && nn < pn1)
              pout[(static_cast<size_t>(mm - pm0) * (pn1 - pn0) + (nn - pn0)) * G + g] = d[r];
          }
        } else {
          const float sg = g < G ? __half2float(sc[t][u]) : 0.0f;
#pragma unroll
          for (int r = 0; r < FR; ++r)
            acc[t][r] = fmaf(static_cast<float>(d[r]), GS ? sg * xsl[u * 32 + d_row(r, h)] : sg, acc[t][r]);
        }
      }
  }
  if (PARTIALS) return;
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int r = 0; r < FR; ++r) red[((t * NW + wave) * FR + r) * 64 + lane] = acc[t][r];
  __syncthreads();
#pragma unroll
  for (int k = 0; k < OPT; ++k) {
    const int o0 = tid + k * NW * 64, o = min(o0, 2 * FR * 64 - 1);
    const int tt = o / (FR * 64), rl = o - tt * FR * 64, r = rl >> 6, l = rl & 63;
    float v = 0.0f;
#pragma unroll
    for (int w = 0; w < NW; ++w) v += red[((tt * NW + w) * FR + r) * 64 + l];
    if (!GS) v *= xsv[k];
    const int mm = d_row(r, l >> 5), nn = r0 + 32 * tt + (l & 31);
    if (o0 == o && mm < M && nn < r1) store_out(y + static_cast<size_t>(mm) * N + nn, v);
  }
}

// ---------------------------------------------------------------- 4-bit GEMV

// The fp16 constants -(1024 + z) and -(64 + z), each twice in a dword, for a
// zero point z in 0..15.
__device__ __forceinline__ uint32_t w4_nz1024(uint32_t z) { return (0xE400u | z) * 0x10001u; }
__device__ __forceinline__ uint32_t w4_nz64(uint32_t z) { return (0xD400u | (z << 4)) * 0x10001u; }

// The eight codes of one packed dword (byte b: code 2b in the low nibble,
// 2b + 1 in the high one) as four fp16 pairs (c_s - z, c_{s+4} - z), s = 0..3,
// exactly: a low nibble under the exponent of 1024 (0x6400 | c is 1024 + c),
// a high nibble, left in place, under the exponent of 64 (0x5400 | c << 4 is
// 64 + c); adding -(1024 + z) or -(64 + z) leaves c - z. One shift, four
// and-or, four packed adds.
__device__ __forceinline__ void w4_pairs_f16(uint32_t w, uint32_t nz1024, uint32_t nz64, h2 out[4]) {
  const uint32_t w8 = w >> 8;
  out[0] = __builtin_bit_cast(h2, and_or(w, 0x000F000Fu, 0x64006400u)) + __builtin_bit_cast(h2, nz1024);
  out[1] = __builtin_bit_cast(h2, and_or(w, 0x00F000F0u, 0x54005400u)) + __builtin_bit_cast(h2, nz64);
  out[2] = __builtin_bit_cast(h2, and_or(w8, 0x000F000Fu, 0x64006400u)) + __builtin_bit_cast(h2, nz1024);
  out[3] = __builtin_bit_cast(h2, and_or(w8, 0x00F000F0u, 0x54005400u)) + __builtin_bit_cast(h2, nz64);
}

// The same as an MFMA B operand: [c0, c4, c1, c5, c2, c6, c3, c7] - z.
__device__ __forceinline__ v8h dequant_w4_f16(uint32_t w, uint32_t nz1024, uint32_t nz64) {
  h2 r[4];
  w4_pairs_f16(w, nz1024, nz64, r);
  const uint32_t r0 = __builtin_bit_cast(uint32_t, r[0]), r1 = __builtin_bit_cast(uint32_t, r[1]);
  const uint32_t r2 = __builtin_bit_cast(uint32_t, r[2]), r3 = __builtin_bit_cast(uint32_t, r[3]);
  return __builtin_bit_cast(v8h, v4u{r0, r1, r2, r3});
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
  v4u cw[MG][2];
  float sc[MG];
  int zc[MG];
  auto load_group = [&](int u, int g) __attribute__((always_inline)) {
    cw[u][0] = *reinterpret_cast<const v4u*>(crow + static_cast<size_t>(g) * 64);
    cw[u][1] = *reinterpret_cast<const v4u*>(crow + static_cast<size_t>(g) * 64 + 32);
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
    const v4u v = reinterpret_cast<const v4u*>(x)[c];
    v4u o;
    o.x = perm_b32(v.z, v.x, 0x05040100u);
    o.y = perm_b32(v.z, v.x, 0x07060302u);
    o.z = perm_b32(v.w, v.y, 0x05040100u);
    o.w = perm_b32(v.w, v.y, 0x07060302u);
    reinterpret_cast<v4u*>(xs)[c] = o;
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
        const uint32_t nzl = w4_nz1024(static_cast<uint32_t>(zc[u])), nzh = w4_nz64(static_cast<uint32_t>(zc[u]));
        const float zf = static_cast<float>(zc[u]);
#pragma unroll
        for (int L = 0; L < 2; ++L) {
          const uint32_t wv[4] = {cw[u][L].x, cw[u][L].y, cw[u][L].z, cw[u][L].w};
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            const v4u araw = *reinterpret_cast<const v4u*>(xa + g * 128 + 64 * L + 8 * s);
            if (BF) {
              const v8bf a = __builtin_bit_cast(v8bf, araw);
              const v8bf b = dequant_w4_bf16(wv[s], zf);
              d = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, d, 0, 0, 0);
            } else {
              const v8h a = __builtin_bit_cast(v8h, araw);
              const v8h b = dequant_w4_f16(wv[s], nzl, nzh);
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

// ---------------------------------------------------------------- 4-bit, 2 <= M <= 16
// Bytes of the skinny 4-bit kernel's LDS before the act-order staging: the
// reduction area (two tiles x NW waves x 4 registers x 64 lanes of fp32) and
// the per-wave scale (2 bytes) and zero-point (1 byte) slices of blk elements,
// rounded up to 16.
__host__ __device__ inline int w4s_lds_head(int nw, int blk) {
  return (2 * nw * 4 * 64 * 4 + 3 * nw * blk + 15) & ~15;
}

// Streaming form for the decode shapes: one workgroup per CU takes rpw weight
// rows (16-row tiles) over the whole K; its NW waves split the groups, GPW
// each. Every load is issued before the first MFMA: scales and zeros, the
// code stream tile by tile, then the activations. MFMA f32_16x16x32 (f16/bf16):
// lane (n, j) = (l % 16, l / 16) holds token row n for A and weight row n of
// the tile for B, columns 32j..32j+31 of each 128-group (16 code bytes, one
// 8-column chunk per MFMA; the activations are permuted inside each chunk to
// the dequantiser's order). The group result is folded with its scale in
// fp32; the waves' sums meet in LDS in a fixed order.
//
// PERM (act order, the mate PR's "Act order" section): the activation gather
// runs inside this kernel. After the scale loads the waves copy the M rows of
// x and the permutation straight into LDS (global -> LDS, no registers), then
// issue the code stream; they wait for the copies only (the code loads stay
// in flight) and build each A operand from LDS, x[m][perm[k']], already in the
// dequantiser's order. K % 512 == 0 and the LDS must hold M rows of x.
//
// SPLIT (K beyond the groups one workgroup's waves can hold): blockIdx.y
// picks a slice of NW * GPW groups, and the workgroup writes its fp32 sums
// (group scales applied) to part[slice][m][n]; splitk_reduce_kernel adds the
// slices in order (split-K as in "Kernel experiments: recorded evidence",
// Tests 21 and 30, and the mate PR's dense kernel).
template <int GPW, int MAXT, bool BF, bool ZP, typename TOut, bool PERM, bool SPLIT>
__global__ __launch_bounds__(PERM ? 1024 : 512) void gemv_w4_skinny_kernel(
    const uint8_t* __restrict__ codes, const uint16_t* __restrict__ wscale,
    const uint8_t* __restrict__ zeros, const uint16_t* __restrict__ x, const int32_t* __restrict__ perm,
    int M, int N, int K, int rpw, TOut* __restrict__ y, float* __restrict__ part) {
  static_assert(!(PERM && SPLIT), "the act-order gather runs without the K split");
  extern __shared__ float red4[];                          // [tile of a pair][wave][reg][lane]
  const int NW = blockDim.x >> 6;
  const int G = K >> 7, KB = K >> 1, ZB = (G + 1) >> 1;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, j = lane >> 4;
  const int r0 = blockIdx.x * rpw;
  const int r1 = min(r0 + rpw, N);
  const int gb = ((SPLIT ? blockIdx.y * NW : 0) + wave) * GPW;

  // Scales and zero bytes of this wave's groups for the workgroup's rows: a
  // (rows x GPW) block per wave, element e = local row e / GPW, group
  // gb + e % GPW, loaded with coalesced small loads (SPL per lane), put in the
  // wave's own LDS slice once the code loads are out and read back in MFMA
  // layout. Only the wave itself touches its slice: no workgroup barrier.
  constexpr int BLK = MAXT * 16 * GPW, SPL = (BLK + 63) / 64;
  uint16_t* ssc = reinterpret_cast<uint16_t*>(red4 + 2 * NW * 4 * 64) + wave * BLK;
  uint8_t* szr = reinterpret_cast<uint8_t*>(reinterpret_cast<uint16_t*>(red4 + 2 * NW * 4 * 64) + NW * BLK) + wave * BLK;
  const int nel = (r1 - r0) * GPW;
  uint16_t sst[SPL];
  uint8_t zst[SPL];
#pragma unroll
  for (int c = 0; c < SPL; ++c) {
    const int e = lane + 64 * c, rr = e / GPW, gc = min(gb + e - rr * GPW, G - 1);
    const size_t row = static_cast<size_t>(r0 + rr);
    sst[c] = e < nel ? wscale[row * G + gc] : 0;
    zst[c] = ZP && e < nel ? zeros[row * ZB + (gc >> 1)] : 0;
  }
  const uint8_t* crow[MAXT];
  int lrow[MAXT];                                          // row within the workgroup's share
#pragma unroll
  for (int t = 0; t < MAXT; ++t) {
    // rows past this workgroup's share read its last row again (same address
    // across the wave) and are never stored
    lrow[t] = min(16 * t + n, r1 - r0 - 1);
    crow[t] = codes + static_cast<size_t>(r0 + lrow[t]) * KB + 16 * j;
  }
  // PERM: LDS after the reduction area and the scale slices holds x row m at
  // byte xo + m * xs and the permutation at xo + M * xs.
  const int xo = w4s_lds_head(NW, BLK), xs = 2 * K + 16;
  if (PERM) {
    const uint32_t lbase = static_cast<uint32_t>(reinterpret_cast<size_t>(red4)) + xo;
    const int per_row = K >> 9;                 // 1 KB pieces of a row
    const int total = M * per_row + (K >> 8);   // and of the 4K-byte permutation
    for (int i = wave; i < total; i += NW) {
      const bool isx = i < M * per_row;
      const int m = isx ? i / per_row : 0;
      const int piece = isx ? i - m * per_row : i - M * per_row;
      const uint8_t* src = isx ? reinterpret_cast<const uint8_t*>(x) + static_cast<size_t>(m) * 2 * K + piece * 1024
                               : reinterpret_cast<const uint8_t*>(perm) + piece * 1024;
      const uint32_t dst = lbase + (isx ? m * xs : M * xs) + piece * 1024;
      lds_dma16(src + lane * 16, __builtin_amdgcn_readfirstlane(dst));
    }
    // every wave's copies go out before any wave's code stream (an execution
    // barrier; it waits for no load): measured at M=8, K=5120, N=13824
    // 15.0-15.2 -> 14.3-14.5 us
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
  }
  __builtin_amdgcn_sched_barrier(0);
  // The code stream, group-tile q = t * GPW + u. Without PERM every load is
  // issued here. With PERM only the first PD are: each later one is issued
  // PD group-tiles ahead of its use, so a wave keeps a few loads in flight
  // while it computes (measured on the 4-bit decode shape, M=8, K=5120,
  // N=13824: 2 ahead 14.6 us, 1 14.7-15.1, 3 14.6-15.3, 4 15.7, 6 16.4, all
  // loads up front 17.2).
  v4u cw[MAXT][GPW];
  constexpr int NQ = MAXT * GPW, PD = PERM ? (NQ < 2 ? NQ : 2) : NQ;
  auto issue = [&](int q) {
    const int t = q / GPW, u = q % GPW;
    cw[t][u] = *reinterpret_cast<const v4u*>(crow[t] + min(gb + u, G - 1) * 64);
    __builtin_amdgcn_sched_barrier(0);
  };
  // A operands: each 8-column chunk in the order [0, 4, 1, 5, 2, 6, 3, 7].
  // Token rows n >= M read row M - 1 (their outputs are never stored).
  v4u a[GPW][4];
  const int mA = min(n, M - 1);
  v4u ain[GPW][4];
  if (!PERM) {
    // Activations first, every wave's ahead of any wave's code stream (an
    // execution barrier; it waits for no load), so the L2-resident rows do
    // not queue behind HBM code loads and tile 0 can start as its codes land
    // (measured on the split form at M=8, K=13824, N=5120: 17.9 -> 17.2 us;
    // without the barrier, activations issued after the code stream had been
    // a little faster than ahead of it).
#pragma unroll
    for (int u = 0; u < GPW; ++u) {
      const int g = min(gb + u, G - 1);
      const v4u* src = reinterpret_cast<const v4u*>(x + static_cast<size_t>(mA) * K + g * 128 + 32 * j);
#pragma unroll
      for (int i = 0; i < 4; ++i) ain[u][i] = src[i];
    }
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int q = 0; q < PD; ++q) issue(q);
  if (!PERM) {
#pragma unroll
    for (int u = 0; u < GPW; ++u)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const v4u v = ain[u][i];
        a[u][i] = v4u{perm_b32(v.z, v.x, 0x05040100u), perm_b32(v.z, v.x, 0x07060302u),
                      perm_b32(v.w, v.y, 0x05040100u), perm_b32(v.w, v.y, 0x07060302u)};
      }
  } else {
    // the copies were issued before the last PD loads (the code stream)
    __builtin_amdgcn_sched_barrier(0);
    wait_vmcnt<PD>();
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int c = 0; c < SPL; ++c) {
    const int e = lane + 64 * c;
    if (e < nel) {
      ssc[e] = sst[c];
      if (ZP) szr[e] = zst[c];
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  // This lane's scales and zero points, read back in one batch.
  uint16_t sreg[MAXT][GPW];
  int zreg[MAXT][GPW];
#pragma unroll
  for (int t = 0; t < MAXT; ++t)
#pragma unroll
    for (int u = 0; u < GPW; ++u) {
      const int gc = min(gb + u, G - 1);
      sreg[t][u] = ssc[lrow[t] * GPW + u];
      zreg[t][u] = ZP ? (szr[lrow[t] * GPW + u] >> (4 * (gc & 1))) & 15 : 8;
    }
  // One group of one tile: the four-MFMA chain over the group's 128 columns,
  // folded with the group scale (groups past the end, from a ragged split of
  // K over the waves, count for nothing).
  auto group_tile = [&](const v4u(&au)[4], int t, int u, float(&acc)[4]) {
    const int g = gb + u;
    const int z = zreg[t][u];
    const uint32_t wv[4] = {cw[t][u].x, cw[t][u].y, cw[t][u].z, cw[t][u].w};
    v4f d = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      if (BF) {
        d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, au[c]),
                                                    dequant_w4_bf16(wv[c], static_cast<float>(z)), d, 0, 0, 0);
      } else {
        d = __builtin_amdgcn_mfma_f32_16x16x32_f16(
            __builtin_bit_cast(v8h, au[c]),
            dequant_w4_f16(wv[c], w4_nz1024(static_cast<uint32_t>(z)), w4_nz64(static_cast<uint32_t>(z))), d, 0, 0, 0);
      }
    }
    const uint16_t sb = sreg[t][u];
    const float sg = g < G ? (BF ? bf16_to_f32(sb) : __half2float(__builtin_bit_cast(__half, sb))) : 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] = fmaf(d[i], sg, acc[i]);
  };
  // PERM: the A operands of the wave's GPW groups come from LDS,
  // x[m][perm[k']] in the dequantiser's order; then tile by tile, group by
  // group, each group-tile's code load is consumed as the one PD ahead is
  // issued. Each tile sums its groups in the order 0..GPW-1.
  float accp[PERM ? MAXT : 1][4];
  if (PERM) {
#pragma unroll
    for (int t = 0; t < MAXT; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) accp[t][i] = 0.0f;
    __syncthreads();   // every wave's copies have landed
    const uint8_t* lx = reinterpret_cast<const uint8_t*>(red4) + xo;
    const uint8_t* xrow = lx + mA * xs;
    // The permutation becomes byte offsets into a row, once per workgroup; an
    // entry outside 0..K-1 reads column K - 1 (the prepare step stores a
    // permutation; this only keeps every LDS read inside the row).
    int32_t* pw = reinterpret_cast<int32_t*>(red4 + xo / 4 + M * xs / 4);
    const uint32_t km = static_cast<uint32_t>(K - 1);
    for (int i = tid; i < (K >> 2); i += NW * 64) {
      const v4i p = reinterpret_cast<const v4i*>(pw)[i];
      reinterpret_cast<v4i*>(pw)[i] = v4i{static_cast<int>(2 * min(static_cast<uint32_t>(p.x), km)),
                                          static_cast<int>(2 * min(static_cast<uint32_t>(p.y), km)),
                                          static_cast<int>(2 * min(static_cast<uint32_t>(p.z), km)),
                                          static_cast<int>(2 * min(static_cast<uint32_t>(p.w), km))};
    }
    __syncthreads();
    const int32_t* pl = pw;
    v4u au[GPW][4];
#pragma unroll
    for (int u = 0; u < GPW; ++u) {
      const int g = min(gb + u, G - 1);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int kb = g * 128 + 32 * j + 8 * i;
        const v4i p0 = *reinterpret_cast<const v4i*>(pl + kb);
        const v4i p1 = *reinterpret_cast<const v4i*>(pl + kb + 4);
        const int pe[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
        uint32_t e[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) e[q] = *reinterpret_cast<const uint16_t*>(xrow + pe[q]);
        au[u][i] = v4u{e[0] | (e[4] << 16), e[1] | (e[5] << 16), e[2] | (e[6] << 16), e[3] | (e[7] << 16)};
      }
    }
#pragma unroll
    for (int t = 0; t < MAXT; ++t)
#pragma unroll
      for (int u = 0; u < GPW; ++u) {
        const int q = t * GPW + u;
        if (q + PD < NQ) issue(q + PD);
        group_tile(au[u], t, u, accp[t]);
      }
  }
  // Tiles in pairs: compute both, then one fixed-order reduction through LDS.
  // Every tile is computed (no branch, so the loads above stay hoisted).
#pragma unroll
  for (int t0 = 0; t0 < MAXT; t0 += 2) {
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const int t = t0 + tt;
      float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
      if (PERM) {
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] = accp[t][i];
      } else {
#pragma unroll
        for (int u = 0; u < GPW; ++u) group_tile(a[u], t, u, acc);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) red4[((tt * NW + wave) * 4 + i) * 64 + lane] = acc[i];
    }
    __syncthreads();
    // 2 tiles x 4 registers x 64 lanes = 512 outputs (16 tokens x 16 rows each)
    for (int o = tid; o < 512; o += NW * 64) {
      const int tt = o >> 8, i = (o >> 6) & 3, l = o & 63;
      float v = 0.0f;
      for (int w = 0; w < NW; ++w) v += red4[((tt * NW + w) * 4 + i) * 64 + l];
      const int mm = 4 * (l >> 4) + i, nn = r0 + 16 * (t0 + tt) + (l & 15);
      if (mm < M && nn < r1) {
        if (SPLIT) part[(static_cast<size_t>(blockIdx.y) * M + mm) * N + nn] = v;
        else store_out(y + static_cast<size_t>(mm) * N + nn, v);
      }
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------- 4-bit, M = 1
// K a multiple of 128, up to 32768. Each wave streams R rows, one 512-byte
// load instruction per 1024 columns (lane l holds the 16 codes of columns
// 16l..16l+15 of each 1024-column chunk, all inside one 128-group); in a last,
// partial chunk the lanes past K load clamped addresses and count zero.
// Past 8 chunks KS = 2 or 4 waves of the workgroup share a row group's K
// (the split-K change of the mate PR's dense kernel: fp32 partials summed in
// a fixed order, here through LDS inside the same launch). The lane's
// 16 activations sit in registers; fp16: the codes become the exact fp16
// values code - zero (magic 1024 trick) and v_dot2_f32_f16 accumulates;
// bf16: codes and activations go through exact fp32 values and the zero point
// is applied as zero * sum(x). The group scale multiplies the fp32 partial.
//
// PERM (act order, the mate PR's "Act order" section: the activation is
// gathered with the permutation that sorted K by group): the gather runs
// inside this kernel. A workgroup loads x and the permutation first, then
// its scales and code stream; while the codes are in flight it
// stages x in LDS, writes x[perm[k']] to a second LDS array and every lane
// reads its activations from there. The barriers wait on LDS traffic only
// (the code loads, issued later, stay in flight across them).
constexpr int kRowW4PermWaves = 4;
constexpr int kRowW4Perm = 2;                 // rows per wave (4 spill into two waves per SIMD)

template <int R, int CH, int KS, bool EXACT, bool BF, bool ZP, typename TOut, bool PERM>
__global__ __launch_bounds__(256) void gemv_w4_row_kernel(
    const uint8_t* __restrict__ codes, const uint16_t* __restrict__ wscale,
    const uint8_t* __restrict__ zeros, const uint16_t* __restrict__ x, const int32_t* __restrict__ perm,
    int N, int K, TOut* __restrict__ y) {
  constexpr int NW = 4, RG = NW / KS;           // waves; row groups per workgroup
  static_assert(KS == 1 || KS == 2 || KS == 4, "a row group takes 1, 2 or 4 waves");
  static_assert(!PERM || (KS == 1 && kRowW4PermWaves == NW), "the act-order gather runs without the K split");
  extern __shared__ __align__(16) uint16_t xstage[];      // PERM: [K] x, then [K] x[perm]; then KS > 1 sums
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ks = wave % KS;                      // this wave's share of K: chunks ks * CH ..
  const int row0 = (blockIdx.x * RG + wave / KS) * R;
  // whole wave; without PERM and without the K split the kernel has no barriers
  if (!PERM && KS == 1 && row0 >= N) return;
  const int KB = K >> 1, G = K >> 7, ZB = (G + 1) >> 1;
  // This lane's columns of chunk cc: 1024 (ks * CH + cc) + 16 lane .. + 15.
  // EXACT: K = 1024 KS CH. Otherwise, in a last, partial chunk (and in chunks
  // past K) the lanes past K read clamped, in-bounds addresses and zero their
  // activations, so they count nothing (no branch around any load;
  // K % 128 == 0 keeps a lane's 16 columns in one group).
  int cbase[CH];
  bool ok[CH];
#pragma unroll
  for (int cc = 0; cc < CH; ++cc) {
    cbase[cc] = (ks * CH + cc) * 1024 + lane * 16;
    ok[cc] = EXACT || cbase[cc] < K;
  }
  const auto xcol = [&](int cc) { return EXACT ? cbase[cc] : min(cbase[cc], K - 16); };
  const auto cbyte = [&](int cc) { return EXACT ? (ks * CH + cc) * 512 + lane * 8 : xcol(cc) >> 1; };
  // Activations of this lane: x[1024c + 16 lane + e], e = 0..15 (PERM: read
  // from LDS after the gather; the staging loads come first).
  v4u xv[CH][2];
  // PERM: 16-byte chunks per thread of x (K / 8 of them) and 32-byte chunks
  // of the permutation (K / 8).
  constexpr int XPT = PERM ? (CH * KS * 128 + 64 * NW - 1) / (64 * NW) : 1;
  const int NX = EXACT ? CH * KS * 128 : K >> 3;
  v4u xin[XPT];
  v4i pin[XPT][2];
  if (PERM) {
#pragma unroll
    for (int i = 0; i < XPT; ++i) {
      const int idx = tid + i * 64 * NW;
      if ((i + 1) * 64 * NW <= NX || idx < NX) {
        xin[i] = reinterpret_cast<const v4u*>(x)[idx];
        pin[i][0] = reinterpret_cast<const v4i*>(perm)[2 * idx];
        pin[i][1] = reinterpret_cast<const v4i*>(perm)[2 * idx + 1];
      }
    }
  } else {
#pragma unroll
    for (int cc = 0; cc < CH; ++cc) {
      const v4u* src = reinterpret_cast<const v4u*>(x + xcol(cc));
      xv[cc][0] = src[0];
      xv[cc][1] = src[1];
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  v2u cw[R][CH];
  // The scales and zero points of a row's groups in this wave's share (8 CH
  // <= 64 of them) in one load each: lane l reads those of group 8 ks CH + l
  // (its zero-point byte holds that group and its neighbour); each lane later
  // takes its own groups' values from there by lane shuffles.
  int sall[R], zall[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const size_t row = static_cast<size_t>(min(row0 + r, N - 1));
    const int gl = min(8 * ks * CH + lane, G - 1);
    sall[r] = wscale[row * G + gl];
    zall[r] = ZP ? zeros[row * ZB + (gl >> 1)] : 0;
  }
  __builtin_amdgcn_sched_barrier(0);
  // the code stream, in the order it is consumed
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const size_t row = static_cast<size_t>(min(row0 + r, N - 1));
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      cw[r][c] = load_stream<v2u>(codes + row * KB + cbyte(c));
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  if (PERM) {
    uint16_t* xr = xstage;
    uint16_t* xg = xstage + K;
#pragma unroll
    for (int i = 0; i < XPT; ++i) {
      const int idx = tid + i * 64 * NW;
      if ((i + 1) * 64 * NW <= NX || idx < NX) reinterpret_cast<v4u*>(xr)[idx] = xin[i];
    }
    __syncthreads();
    // x[perm[k']] for 8 consecutive k', written in the pair order of the
    // decode below: (x_s, x_{s+4}) for s = 0..3 of each 8.
#pragma unroll
    for (int i = 0; i < XPT; ++i) {
      const int idx = tid + i * 64 * NW;
      if ((i + 1) * 64 * NW <= NX || idx < NX) {
        // an entry outside 0..K-1 reads column K - 1 (the prepare step stores a
        // permutation; this only keeps every LDS read inside x)
        const uint32_t km = static_cast<uint32_t>(K - 1);
        const int pe[8] = {pin[i][0].x, pin[i][0].y, pin[i][0].z, pin[i][0].w,
                           pin[i][1].x, pin[i][1].y, pin[i][1].z, pin[i][1].w};
        uint32_t e[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) e[j] = xr[min(static_cast<uint32_t>(pe[j]), km)];
        reinterpret_cast<v4u*>(xg)[idx] =
            v4u{e[0] | (e[4] << 16), e[1] | (e[5] << 16), e[2] | (e[6] << 16), e[3] | (e[7] << 16)};
      }
    }
    __syncthreads();
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const v4u* src = reinterpret_cast<const v4u*>(xg + xcol(c));
      xv[c][0] = src[0];
      xv[c][1] = src[1];
    }
  } else {
    // keep the activation permutes below the code loads
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      asm volatile("" : "+v"(xv[c][0]));
      asm volatile("" : "+v"(xv[c][1]));
    }
  }
  if (!EXACT) {
#pragma unroll
    for (int c = 0; c < CH; ++c)
      if (!ok[c]) xv[c][0] = xv[c][1] = v4u{0, 0, 0, 0};
  }
  // Per group (lane l = group l): the fp32 scale, the zero point and, for
  // fp16, the packed fp16 constants -(1024 + z) and -(64 + z) of the decode
  // below; each lane then takes those of its chunk's group.
  float sv[R][CH];
  int zv[R][CH];
  uint32_t nzl[R][CH], nzh[R][CH];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const uint16_t sb = static_cast<uint16_t>(sall[r]);
    const float sf = BF ? bf16_to_f32(sb) : __half2float(__builtin_bit_cast(__half, sb));
    const uint32_t zg = ZP ? (static_cast<uint32_t>(zall[r]) >> (4 * (lane & 1))) & 15u : 8u;   // 8 ks CH is even
    const uint32_t pl = w4_nz1024(zg), ph = w4_nz64(zg);
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int g = 8 * c + (lane >> 3);          // lane holding this chunk's group
      sv[r][c] = __shfl(sf, g);
      if (BF) {
        zv[r][c] = ZP ? __shfl(static_cast<int>(zg), g) : 8;
      } else if (ZP) {
        nzl[r][c] = static_cast<uint32_t>(__shfl(static_cast<int>(pl), g));
        nzh[r][c] = static_cast<uint32_t>(__shfl(static_cast<int>(ph), g));
      } else {
        nzl[r][c] = pl;
        nzh[r][c] = ph;
      }
    }
  }
  float acc[R];
#pragma unroll
  for (int r = 0; r < R; ++r) acc[r] = 0.0f;
  if (!BF) {
    // x pairs in the order the code pairs come out: (x_s, x_{s+4}) of each 8
    // (PERM: the gather wrote them in that order).
    h2 xp[CH][8];
#pragma unroll
    for (int c = 0; c < CH; ++c) {
#pragma unroll
      for (int d = 0; d < 2; ++d) {
        const v4u v = xv[c][d];
        if (PERM) {
          // (components go through named scalars: this compiler bit-casts a
          // vector component expression such as v.y as if it were v.x)
          const uint32_t v0 = v.x, v1 = v.y, v2 = v.z, v3 = v.w;
          xp[c][4 * d + 0] = __builtin_bit_cast(h2, v0);
          xp[c][4 * d + 1] = __builtin_bit_cast(h2, v1);
          xp[c][4 * d + 2] = __builtin_bit_cast(h2, v2);
          xp[c][4 * d + 3] = __builtin_bit_cast(h2, v3);
        } else {
          xp[c][4 * d + 0] = __builtin_bit_cast(h2, perm_b32(v.z, v.x, 0x05040100u));
          xp[c][4 * d + 1] = __builtin_bit_cast(h2, perm_b32(v.z, v.x, 0x07060302u));
          xp[c][4 * d + 2] = __builtin_bit_cast(h2, perm_b32(v.w, v.y, 0x05040100u));
          xp[c][4 * d + 3] = __builtin_bit_cast(h2, perm_b32(v.w, v.y, 0x07060302u));
        }
      }
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
#pragma unroll
      for (int c = 0; c < CH; ++c) {
        const uint32_t wv[2] = {cw[r][c].x, cw[r][c].y};
        float p = 0.0f;
#pragma unroll
        for (int d = 0; d < 2; ++d) {
          h2 cz[4];
          w4_pairs_f16(wv[d], nzl[r][c], nzh[r][c], cz);
#pragma unroll
          for (int s = 0; s < 4; ++s) p = __builtin_amdgcn_fdot2(cz[s], xp[c][4 * d + s], p, false);
        }
        acc[r] = fmaf(sv[r][c], p, acc[r]);
      }
    }
  } else {
    float xf[CH][16];
    float xsum[CH];
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const uint32_t xw[8] = {xv[c][0].x, xv[c][0].y, xv[c][0].z, xv[c][0].w,
                              xv[c][1].x, xv[c][1].y, xv[c][1].z, xv[c][1].w};
      xsum[c] = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        // dword e = 4d + s holds elements 8d + 2s, 8d + 2s + 1 (PERM: the
        // pair-ordered gather put 8d + s and 8d + s + 4 there)
        const int d = e >> 2, s4 = e & 3;
        const int lo = PERM ? 8 * d + s4 : 2 * e, hi = PERM ? 8 * d + s4 + 4 : 2 * e + 1;
        xf[c][lo] = __uint_as_float(xw[e] << 16);
        xf[c][hi] = __uint_as_float(xw[e] & 0xFFFF0000u);
      }
#pragma unroll
      for (int e = 0; e < 16; ++e) xsum[c] += xf[c][e];
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
#pragma unroll
      for (int c = 0; c < CH; ++c) {
        const uint32_t wv[2] = {cw[r][c].x, cw[r][c].y};
        float p = 0.0f;
#pragma unroll
        for (int d = 0; d < 2; ++d)
#pragma unroll
          for (int e = 0; e < 8; ++e)
            p = fmaf(static_cast<float>((wv[d] >> (4 * e)) & 15u), xf[c][8 * d + e], p);
        p = fmaf(-static_cast<float>(zv[r][c]), xsum[c], p);
        acc[r] = fmaf(sv[r][c], p, acc[r]);
      }
    }
  }
  if (KS == 1) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const float v = wave_sum(acc[r]);
      if (lane == r && row0 + r < N) store_out(y + row0 + r, v);
    }
  } else {
    // the KS waves of a row group meet in LDS and are added in share order
    float* part = reinterpret_cast<float*>(xstage);
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const float v = wave_sum(acc[r]);
      if (lane == 0) part[wave * R + r] = v;
    }
    __syncthreads();
    if (ks == 0 && lane < R && row0 + lane < N) {
      float v = 0.0f;
#pragma unroll
      for (int k2 = 0; k2 < KS; ++k2) v += part[(wave + k2) * R + lane];
      store_out(y + row0 + lane, v);
    }
  }
}

int fold_for(int64_t m) { return m <= 1 ? 1 : (m <= 8 ? 4 : (m <= 16 ? 8 : 16)); }
int waves_for(int64_t groups) { return groups >= 16 ? 8 : 4; }

// Rows per wave in the M = 1 kernels (measured on the decode shapes: fewer rows
// per wave put more waves in flight; one row per wave pays the activation
// transpose too often).
constexpr int kRowT2 = 2;
constexpr int kRowW4 = 2;

bool t2_row_ok(int64_t m, int64_t k) { return m == 1 && k <= 4 * 4096; }
// The M = 1 4-bit kernel takes K in chunks of 1024 columns, the last one
// possibly partial (K % 128 == 0), at most 8 chunks per wave; past 8 chunks
// 2 or 4 waves share a row group's K.
bool w4_row_ok(int64_t m, int64_t k) { return m == 1 && k > 0 && k % 128 == 0 && k <= 4 * 8 * 1024; }
bool w4_row_perm_ok(int64_t m, int64_t k) { return m == 1 && k > 0 && k % 128 == 0 && k <= 8 * 1024; }
int w4_row_split(int64_t k) {
  const int64_t c = (k + 1023) / 1024;
  if (c <= 8) return 1;
  return c <= 16 ? 2 : 4;
}
int w4_row_chunks(int64_t k) {
  const int ks = w4_row_split(k);
  return static_cast<int>(((k + 1023) / 1024 + ks - 1) / ks);
}


// Each wave reads the whole activation row (4 KB per 4096 columns) for its R
// rows of 1 KB each per 4096 columns: at R = 2 that is twice the code bytes.
// With many rows (N >= 16384) there are waves to spare, and four rows per wave
// halve that traffic (measured on K = 8192, N = 28672: 4 rows 13.6-14.3 us,
// 2 rows 15.7-16.2 us, 8 rows 15.3-15.5 us).
constexpr int kRowT2Wide = 4;
constexpr int kWideRows = 16384;

template <int CH, typename TOut, bool PARTIALS, bool GS, typename TX = int8_t>
void t2_row_go(const bpw_weights& w, const TX* q, const float* xs, TOut* y, int32_t* pout,
               int pn0, int pn1, hipStream_t s) {
  const int n = static_cast<int>(w.n), k = static_cast<int>(w.k);
  constexpr int nw = std::is_same<TX, int8_t>::value ? 4 : kFusedWaves;
  const int rows = n >= kWideRows ? kRowT2Wide : kRowT2;
  const unsigned blocks = static_cast<unsigned>(((n + rows - 1) / rows + nw - 1) / nw);
  if (n >= kWideRows)
    gemv_t2_row_kernel<kRowT2Wide, CH, TOut, PARTIALS, GS, TX><<<blocks, 64 * nw, 0, s>>>(
        static_cast<const uint8_t*>(w.codes), static_cast<const __half*>(w.scales), q, xs, n, k, y,
        pout, pn0, pn1);
  else
    gemv_t2_row_kernel<kRowT2, CH, TOut, PARTIALS, GS, TX><<<blocks, 64 * nw, 0, s>>>(
        static_cast<const uint8_t*>(w.codes), static_cast<const __half*>(w.scales), q, xs, n, k, y,
        pout, pn0, pn1);
}

// The complete one-token call: 16-bit or fp32 activations quantised inside
// the row kernel.
template <typename TOut, typename TX>
hipError_t t2_row_fused(const bpw_weights& w, const TX* x, TOut* y, hipStream_t s) {
  switch ((w.k + 4095) / 4096) {
    case 1: t2_row_go<1, TOut, false, false, TX>(w, x, nullptr, y, nullptr, 0, 0, s); break;
    case 2: t2_row_go<2, TOut, false, false, TX>(w, x, nullptr, y, nullptr, 0, 0, s); break;
    case 3: t2_row_go<3, TOut, false, false, TX>(w, x, nullptr, y, nullptr, 0, 0, s); break;
    default: t2_row_go<4, TOut, false, false, TX>(w, x, nullptr, y, nullptr, 0, 0, s); break;
  }
  return hipGetLastError();
}

template <typename TOut>
hipError_t t2_fused_dispatch(const bpw_weights& w, const void* x, int x_dtype, TOut* y, hipStream_t s) {
  switch (x_dtype) {
    case BPW_F32: return t2_row_fused(w, static_cast<const float*>(x), y, s);
    case BPW_F16: return t2_row_fused(w, static_cast<const __half*>(x), y, s);
    default: return t2_row_fused(w, static_cast<const uint16_t*>(x), y, s);
  }
}

template <typename TOut, bool PARTIALS, bool GS = false>
hipError_t t2_row(const bpw_weights& w, const int8_t* q, const float* xs, TOut* y, int32_t* pout,
                  int pn0, int pn1, hipStream_t s) {
  switch ((w.k + 4095) / 4096) {
    case 1: t2_row_go<1, TOut, PARTIALS, GS>(w, q, xs, y, pout, pn0, pn1, s); break;
    case 2: t2_row_go<2, TOut, PARTIALS, GS>(w, q, xs, y, pout, pn0, pn1, s); break;
    case 3: t2_row_go<3, TOut, PARTIALS, GS>(w, q, xs, y, pout, pn0, pn1, s); break;
    default: t2_row_go<4, TOut, PARTIALS, GS>(w, q, xs, y, pout, pn0, pn1, s); break;
  }
  return hipGetLastError();
}

// Compute units of the current device (the skinny kernel runs one workgroup per
// CU); queried once per device. Callers on several host threads may race to
// fill an entry; they store the same value.
int cu_count() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int c = cached[dev].load(std::memory_order_relaxed);
  if (c == 0) {
    if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || c <= 0) c = 256;
    cached[dev].store(c, std::memory_order_relaxed);
  }
  return c;
}

// The skinny kernel holds a wave's whole K slice in registers: up to 32
// groups (16 waves of 2) without spilling. Longer K goes to the long kernel.
bool t2_skinny_ok(int64_t m, int64_t k) { return m >= 2 && m <= 32 && k <= 128 * 32; }
bool t2_long_ok(int64_t m, int64_t k) { return m >= 1 && m <= 32; }

// Rows per workgroup: the rows split evenly over the CUs, at least 16, at most
// four 32-row tiles.
int skinny_rpw(int n) {
  const int cus = cu_count();
  int rpw = (n + cus - 1) / cus;
  rpw = max(16, (rpw + 7) & ~7);
  return min(rpw, 128);
}

template <int NW, int GPW, int MAXT, typename TOut, bool PARTIALS, bool GS>
void t2_skinny_go(const bpw_weights& w, const int8_t* q, const float* xs, int m, int rpw, TOut* y,
                  int32_t* pout, int pm0, int pm1, int pn0, int pn1, int wg0, int nwg, hipStream_t s) {
  const uint8_t* codes = static_cast<const uint8_t*>(w.codes);
  const __half* sc = static_cast<const __half*>(w.scales);
  const int n = static_cast<int>(w.n), k = static_cast<int>(w.k);
  const size_t gs_lds = GS ? 4ull * NW * GPW * 32 : 0;     // activation group scales, per wave
  if (m <= 16) {
    auto kern = gemv_t2_skinny_kernel<NW, GPW, MAXT, 8, TOut, PARTIALS, GS>;
    const size_t lds = 2ull * NW * 8 * 64 * 4 + gs_lds;
    allow_lds(kern, lds);
    kern<<<nwg, NW * 64, lds, s>>>(codes, sc, q, xs, m, n, k, rpw, y, pout, pm0, pm1, pn0, pn1, wg0, nullptr);
  } else {
    // (the dispatcher sends scaled-by-group products above 16 rows to the long
    // kernel: that form is not built, it would spill)
    constexpr int FR = GS ? 8 : 16;
    auto kern = gemv_t2_skinny_kernel<NW, GPW, MAXT, FR, TOut, PARTIALS, GS>;
    const size_t lds = 2ull * NW * FR * 64 * 4 + gs_lds;
    allow_lds(kern, lds);
    kern<<<nwg, NW * 64, lds, s>>>(codes, sc, q, xs, m, n, k, rpw, y, pout, pm0, pm1, pn0, pn1, wg0, nullptr);
  }
}

template <typename TOut, bool PARTIALS, bool GS = false>
hipError_t t2_skinny(const bpw_weights& w, const int8_t* q, const float* xs, int m, TOut* y,
                     int32_t* pout, int pm0, int pm1, int pn0, int pn1, hipStream_t s) {
  const int n = static_cast<int>(w.n), g = static_cast<int>(w.k / 128);
  const int rpw = skinny_rpw(n);
  // waves split K: 16 waves of up to 2 groups from 16 groups up, 8 below
  const int nw = g >= 16 ? 16 : 8;
  const int gpw = (g + nw - 1) / nw;
  // workgroups covering weight rows [pn0, pn1) (the whole matrix for a product)
  const int wg0 = PARTIALS ? pn0 / rpw : 0;
  const int nwg = PARTIALS ? (pn1 - 1) / rpw - wg0 + 1 : (n + rpw - 1) / rpw;
  const bool two = rpw <= 64;
#define BPW_SK(NW_, GPW_)                                                                          \
  if (nw == NW_ && gpw == GPW_) {                                                                 \
    if (two) t2_skinny_go<NW_, GPW_, 2, TOut, PARTIALS, GS>(w, q, xs, m, rpw, y, pout, pm0, pm1, pn0, pn1, wg0, nwg, s); \
    else t2_skinny_go<NW_, GPW_, 4, TOut, PARTIALS, GS>(w, q, xs, m, rpw, y, pout, pm0, pm1, pn0, pn1, wg0, nwg, s);     \
    return hipGetLastError();                                                                     \
  }
  BPW_SK(8, 1) BPW_SK(8, 2) BPW_SK(16, 1) BPW_SK(16, 2)
#undef BPW_SK
  return hipErrorInvalidValue;
}

// y[m][n] = x_scale[m] * (part[0][m][n] + part[1][m][n] + ...), slices in
// order; without x_scale (4-bit weights) the sum itself.
template <typename TOut>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ part, int splits, int M,
                                                            int N, const float* __restrict__ x_scale,
                                                            TOut* __restrict__ y) {
  const size_t total = static_cast<size_t>(M) * N;
  for (size_t i = blockIdx.x * 256ull + threadIdx.x; i < total; i += gridDim.x * 256ull) {
    float v = part[i];
    for (int sl = 1; sl < splits; ++sl) v += part[sl * total + i];
    store_out(y + i, x_scale ? v * x_scale[i / N] : v);
  }
}

// Split-K for 2 <= M <= 32 beyond 32 groups ("Kernel experiments: recorded
// evidence", Tests 21 and 30: more blocks for small-output shapes, partial sums
// added in a fixed order by a second kernel): slices of 32 groups (16 waves of
// 2) side by side, rows per workgroup chosen so that row blocks x slices fill
// the CUs about once.
int t2_splits(int64_t k) { return static_cast<int>((k / 128 + 31) / 32); }
bool t2_split_ok(int64_t m, int64_t k) { return m >= 2 && m <= 32 && k > 128 * 32; }

template <typename TOut>
hipError_t t2_split(const bpw_weights& w, const int8_t* q, const float* xs, int m, TOut* y, float* part,
                    hipStream_t s) {
  const int n = static_cast<int>(w.n), k = static_cast<int>(w.k);
  const int splits = t2_splits(k);
  // the fewest rows per workgroup (a multiple of 8, 16..128) whose row blocks
  // times slices still fit one workgroup per CU; 128 if none does
  const int cus = cu_count();
  int rpw = 16;
  while (rpw < 128 && static_cast<int64_t>((n + rpw - 1) / rpw) * splits > cus) rpw += 8;
  const int nwg = (n + rpw - 1) / rpw;
  const uint8_t* codes = static_cast<const uint8_t*>(w.codes);
  const __half* sc = static_cast<const __half*>(w.scales);
  const dim3 grid(nwg, splits);
  auto go = [&](auto kern, int fr) {
    const size_t lds = 2ull * 16 * fr * 64 * 4;
    allow_lds(kern, lds);
    kern<<<grid, 16 * 64, lds, s>>>(codes, sc, q, xs, m, n, k, rpw, y, nullptr, 0, 0, 0, 0, 0, part);
  };
  if (m <= 16) {
    if (rpw <= 64) go(gemv_t2_skinny_kernel<16, 2, 2, 8, TOut, false, false, true>, 8);
    else go(gemv_t2_skinny_kernel<16, 2, 4, 8, TOut, false, false, true>, 8);
  } else {
    if (rpw <= 64) go(gemv_t2_skinny_kernel<16, 2, 2, 16, TOut, false, false, true>, 16);
    else go(gemv_t2_skinny_kernel<16, 2, 4, 16, TOut, false, false, true>, 16);
  }
  const size_t total = static_cast<size_t>(m) * n;
  const int rblocks = static_cast<int>(std::min<size_t>((total + 255) / 256, 4096));
  splitk_reduce_kernel<TOut><<<rblocks, 256, 0, s>>>(part, splits, m, n, xs, y);
  return hipGetLastError();
}

template <int NW, int FR, typename TOut, bool PARTIALS, bool GS>
void t2_long_go(const bpw_weights& w, const int8_t* q, const float* xs, int m, int rpw, TOut* y,
                int32_t* pout, int pm0, int pm1, int pn0, int pn1, int wg0, int nwg, hipStream_t s) {
  auto kern = gemv_t2_long_kernel<NW, FR, TOut, PARTIALS, GS>;
  const size_t lds = 2ull * NW * FR * 64 * 4 + (GS ? 4ull * NW * 64 : 0);
  allow_lds(kern, lds);
  kern<<<nwg, NW * 64, lds, s>>>(static_cast<const uint8_t*>(w.codes), static_cast<const __half*>(w.scales), q,
                                 xs, m, static_cast<int>(w.n), static_cast<int>(w.k), rpw, y, pout, pm0, pm1,
                                 pn0, pn1, wg0);
}

template <typename TOut, bool PARTIALS, bool GS = false>
hipError_t t2_long(const bpw_weights& w, const int8_t* q, const float* xs, int m, TOut* y,
                   int32_t* pout, int pm0, int pm1, int pn0, int pn1, hipStream_t s) {
  const int n = static_cast<int>(w.n);
  const int rpw = min(skinny_rpw(n), 64);                  // two 32-row tiles
  const int wg0 = PARTIALS ? pn0 / rpw : 0;
  const int nwg = PARTIALS ? (pn1 - 1) / rpw - wg0 + 1 : (n + rpw - 1) / rpw;
  // 16 waves (128 VGPRs each) while the accumulators hold 8 registers, 8
  // waves for 16 (more would spill)
  if (m <= 16) t2_long_go<16, 8, TOut, PARTIALS, GS>(w, q, xs, m, rpw, y, pout, pm0, pm1, pn0, pn1, wg0, nwg, s);
  else t2_long_go<8, 16, TOut, PARTIALS, GS>(w, q, xs, m, rpw, y, pout, pm0, pm1, pn0, pn1, wg0, nwg, s);
  return hipGetLastError();
}

// M = 1 up to K = 16384: the row kernel; M = 2..32 up to 32 groups: the
// skinny kernel; any other M <= 32: the long-K kernel. The same routing with
// per-(row, group) activation scales.
// The staged kernel: 2 <= M <= 16, K a multiple of 1024 up to 4096 (the
// scale rows and code rows then split into whole 16-byte copies), 16-byte
// aligned activations and code plane, and (group activation scales) a
// 16-byte aligned x_scale.
bool t2_stage_ok(int64_t m, int64_t k, const void* q, const void* codes, const void* xs, bool gs) {
  return m >= 2 && m <= 16 && k % 1024 == 0 && k <= 4096 && reinterpret_cast<uintptr_t>(q) % 16 == 0 &&
         reinterpret_cast<uintptr_t>(codes) % 16 == 0 && (!gs || reinterpret_cast<uintptr_t>(xs) % 16 == 0);
}

template <typename TOut, bool PARTIALS, bool GS>
hipError_t t2_stage(const bpw_weights& w, const int8_t* q, const float* xs, int m, TOut* y, int32_t* pout,
                    int pm0, int pm1, int pn0, int pn1, hipStream_t s) {
  const int n = static_cast<int>(w.n), k = static_cast<int>(w.k), g = k / 128;
  const int cus = cu_count();
  int rpw = (n + cus - 1) / cus;
  rpw = min(16 * kStageTiles, max(16, (rpw + 7) & ~7));
  const int gpw = (g + kStageWaves - 1) / kStageWaves;      // 1 or 2
  const int xs_bytes = PARTIALS ? 0 : (GS ? m * g * 4 : m * 4);
  const T2StageLds L = t2_stage_lds(k, g, gpw, xs_bytes);
  const unsigned blocks = static_cast<unsigned>((n + rpw - 1) / rpw);
  auto go = [&](auto kern) {
    allow_lds(kern, L.total);
    kern<<<blocks, 64 * kStageWaves, L.total, s>>>(static_cast<const uint8_t*>(w.codes),
                                                     static_cast<const __half*>(w.scales), q, xs, m, n, k, rpw, y,
                                                     pout, pm0, pm1, pn0, pn1, nullptr);
  };
  if (gpw == 1) go(gemv_t2_stage_kernel<1, TOut, PARTIALS, GS>);
  else go(gemv_t2_stage_kernel<2, TOut, PARTIALS, GS>);
  return hipGetLastError();
}

// The staged kernel over K slices of 32 groups (2 <= M <= 16, K > 4096 a
// multiple of 1024, row scales), then the fixed-order reduce of the slices.
// Rows per workgroup: the fewest (a multiple of 8, 16..64) whose row blocks
// times slices fit one workgroup per CU.
bool t2_stage_split_ok(int64_t m, int64_t k, const void* q, const void* codes) {
  return m >= 2 && m <= 16 && k > 4096 && k % 1024 == 0 && reinterpret_cast<uintptr_t>(q) % 16 == 0 &&
         reinterpret_cast<uintptr_t>(codes) % 16 == 0;
}

template <typename TOut>
hipError_t t2_stage_split(const bpw_weights& w, const int8_t* q, const float* xs, int m, TOut* y, float* part,
                          hipStream_t s) {
  const int n = static_cast<int>(w.n), k = static_cast<int>(w.k);
  const int splits = t2_splits(k);                          // slices of 32 groups
  const int cus = cu_count();
  int rpw = 16;
  while (rpw < 16 * kStageTiles && static_cast<int64_t>((n + rpw - 1) / rpw) * splits > cus) rpw += 8;
  const T2StageLds L = t2_stage_lds(4096, 32, 2, 0);
  const dim3 grid((n + rpw - 1) / rpw, splits);
  auto kern = gemv_t2_stage_kernel<2, TOut, false, false, true>;
  allow_lds(kern, L.total);
  kern<<<grid, 64 * kStageWaves, L.total, s>>>(static_cast<const uint8_t*>(w.codes),
                                               static_cast<const __half*>(w.scales), q, xs, m, n, k, rpw, y,
                                               nullptr, 0, 0, 0, 0, part);
  const size_t total = static_cast<size_t>(m) * n;
  const int rblocks = static_cast<int>(std::min<size_t>((total + 255) / 256, 4096));
  splitk_reduce_kernel<TOut><<<rblocks, 256, 0, s>>>(part, splits, m, n, xs, y);
  return hipGetLastError();
}

template <typename TOut>
hipError_t t2_dispatch(const bpw_weights& w, const int8_t* q, const float* xs, int m, TOut* y,
                       bool gs, float* part, hipStream_t s) {
  if (t2_stage_ok(m, w.k, q, w.codes, xs, gs)) {
    if (gs) return t2_stage<TOut, false, true>(w, q, xs, m, y, nullptr, 0, 0, 0, 0, s);
    return t2_stage<TOut, false, false>(w, q, xs, m, y, nullptr, 0, 0, 0, 0, s);
  }
  if (gs) {
    if (t2_row_ok(m, w.k)) return t2_row<TOut, false, true>(w, q, xs, y, nullptr, 0, 0, s);
    // (above 16 rows the skinny kernel's four-tile form would spill with the scales)
    if (m <= 16 && t2_skinny_ok(m, w.k)) return t2_skinny<TOut, false, true>(w, q, xs, m, y, nullptr, 0, 0, 0, 0, s);
    if (t2_long_ok(m, w.k)) return t2_long<TOut, false, true>(w, q, xs, m, y, nullptr, 0, 0, 0, 0, s);
    return hipErrorInvalidValue;
  }
  if (t2_row_ok(m, w.k)) return t2_row<TOut, false>(w, q, xs, y, nullptr, 0, 0, s);
  if (t2_skinny_ok(m, w.k)) return t2_skinny<TOut, false>(w, q, xs, m, y, nullptr, 0, 0, 0, 0, s);
  if (part && t2_stage_split_ok(m, w.k, q, w.codes)) return t2_stage_split<TOut>(w, q, xs, m, y, part, s);
  if (part && t2_split_ok(m, w.k)) return t2_split<TOut>(w, q, xs, m, y, part, s);
  if (t2_long_ok(m, w.k)) return t2_long<TOut, false>(w, q, xs, m, y, nullptr, 0, 0, 0, 0, s);
  return hipErrorInvalidValue;
}

template <int NW, int FOLD, bool BF, bool ZP, typename TOut>
hipError_t w4_go(const bpw_weights& w, const uint16_t* x, int m, TOut* y, hipStream_t s) {
  const int n = static_cast<int>(w.n), k = static_cast<int>(w.k);
  const size_t stage = static_cast<size_t>(m) * k * 2;
  const size_t red = static_cast<size_t>(NW) * FOLD * 64 * 4;
  const size_t lds = stage > red ? stage : red;
  dim3 grid((n + kRows - 1) / kRows), block(NW * 64);
  allow_lds(gemv_w4_kernel<NW, FOLD, BF, ZP, TOut>, lds);
  gemv_w4_kernel<NW, FOLD, BF, ZP, TOut><<<grid, block, lds, s>>>(
      static_cast<const uint8_t*>(w.codes), static_cast<const uint16_t*>(w.scales),
      static_cast<const uint8_t*>(w.zeros), x, m, n, k, y);
  return hipGetLastError();
}

// 16..48 groups: 4..6 per wave (6 spills a few registers with zero points,
// still far ahead of the LDS-tiled kernel, whose staging does not fit M * K
// at these sizes)
bool w4_skinny_ok(int64_t m, int64_t k) { return m >= 2 && m <= 16 && k / 128 >= 16 && k / 128 <= 48; }
bool w4_split_ok(int64_t m, int64_t k) { return m >= 2 && m <= 16 && k / 128 > 48; }

// LDS of the act-order staging: M rows of x (2K bytes + 16 of padding each)
// and the 4K-byte permutation.
size_t w4s_perm_lds(int64_t m, int64_t k) { return static_cast<size_t>(m) * (2 * k + 16) + 4 * k; }

template <int GPW, int MAXT, bool BF, bool ZP, bool PERM, typename TOut, bool SPLIT = false>
void w4_skinny_go(const bpw_weights& w, const uint16_t* x, int m, int rpw, int nw, TOut* y, hipStream_t s,
                  int splits = 1, float* part = nullptr) {
  const int n = static_cast<int>(w.n), k = static_cast<int>(w.k);
  auto kern = gemv_w4_skinny_kernel<GPW, MAXT, BF, ZP, TOut, PERM, SPLIT>;
  const size_t lds = w4s_lds_head(nw, MAXT * 16 * GPW) + (PERM ? w4s_perm_lds(m, k) : 0);
  allow_lds(kern, lds);
  kern<<<dim3((n + rpw - 1) / rpw, splits), nw * 64, lds, s>>>(
      static_cast<const uint8_t*>(w.codes), static_cast<const uint16_t*>(w.scales),
      static_cast<const uint8_t*>(w.zeros), x, w.perm, m, n, k, rpw, y, part);
}

// Launch shape of the skinny 4-bit kernel: rows split evenly over the CUs
// (multiple of 8, 16..64: at most four 16-row tiles), up to 8 waves of 4..6
// groups (16 <= groups <= 48).
struct W4SkinnyShape {
  int rpw, nw, gpw, maxt;
};

W4SkinnyShape w4_skinny_shape(int64_t n, int64_t k, bool perm) {
  const int g = static_cast<int>(k / 128);
  const int cus = cu_count();
  int rpw = static_cast<int>((n + cus - 1) / cus);
  rpw = min(64, max(16, (rpw + 7) & ~7));
  // act order: 3 groups per wave and up to 16 waves (the gathered operands
  // are built group by group, so a wave needs fewer registers and more waves
  // share the CU)
  const int nw = perm ? (g + 2) / 3 : min(8, (g + 3) / 4);
  return {rpw, nw, (g + nw - 1) / nw, rpw <= 32 ? 2 : 4};
}

template <bool BF, bool ZP, bool PERM, typename TOut>
hipError_t w4_skinny(const bpw_weights& w, const uint16_t* x, int m, TOut* y, hipStream_t s) {
  const W4SkinnyShape sh = w4_skinny_shape(w.n, w.k, PERM);
#define BPW_W4S(GPW_)                                                                            \
  if (sh.gpw == GPW_) {                                                                         \
    if (sh.maxt == 2) w4_skinny_go<GPW_, 2, BF, ZP, PERM>(w, x, m, sh.rpw, sh.nw, y, s);        \
    else w4_skinny_go<GPW_, 4, BF, ZP, PERM>(w, x, m, sh.rpw, sh.nw, y, s);                     \
    return hipGetLastError();                                                                   \
  }
  if (PERM) {
    BPW_W4S(3)
  } else {
    BPW_W4S(4) BPW_W4S(5) BPW_W4S(6)
  }
#undef BPW_W4S
  return hipErrorInvalidValue;
}

// Split-K of the skinny kernel for 2 <= M <= 16 beyond 48 groups: slices of
// at most 16 groups (up to 4 waves of 4), as even as 4-group waves allow, and
// 32 rows per workgroup, then a fixed-order reduce of the slices. Measured on
// K=13824, N=5120, M=8 (108 groups): 16-group slices and 32 rows 18.0 us;
// 16-group slices with 64 rows 19.6; 32-group slices with 32 rows 22.6, with
// 16 rows 30.9, with 64 rows 25.0; 12-group slices 20.1; 8-group 22.1.
struct W4SplitShape {
  int splits, nw, rpw;
};

int w4_split_waves(int64_t k) {
  const int g = static_cast<int>(k / 128), s0 = (g + 15) / 16;
  return ((g + s0 - 1) / s0 + 3) / 4;                            // 4-group waves per slice
}
int w4_splits(int64_t k) { return static_cast<int>((k / 128 + 4 * w4_split_waves(k) - 1) / (4 * w4_split_waves(k))); }

W4SplitShape w4_split_shape(int64_t k) { return {w4_splits(k), w4_split_waves(k), 32}; }

template <bool BF, bool ZP, typename TOut>
hipError_t w4_split(const bpw_weights& w, const uint16_t* x, int m, TOut* y, float* part, hipStream_t s) {
  const W4SplitShape sh = w4_split_shape(w.k);
  w4_skinny_go<4, 2, BF, ZP, false, TOut, true>(w, x, m, sh.rpw, sh.nw, y, s, sh.splits, part);
  const int n = static_cast<int>(w.n);
  const size_t total = static_cast<size_t>(m) * n;
  const int rblocks = static_cast<int>(std::min<size_t>((total + 255) / 256, 4096));
  splitk_reduce_kernel<TOut><<<rblocks, 256, 0, s>>>(part, sh.splits, m, n, nullptr, y);
  return hipGetLastError();
}

// The skinny kernel gathers the act-order activation itself when K is a
// multiple of 512 and M rows of x fit in the LDS beside its other arrays.
bool w4_skinny_perm_ok(int64_t m, int64_t k) {
  if (!w4_skinny_ok(m, k) || k % 512 != 0) return false;
  const W4SkinnyShape sh = w4_skinny_shape(1 << 20, k, true);   // the largest tile count
  return w4s_lds_head(sh.nw, 4 * 16 * sh.gpw) + w4s_perm_lds(m, k) <= 160 * 1024;
}

template <int CH, int KS, bool EXACT, bool BF, bool ZP, typename TOut>
void w4_row_go(const bpw_weights& w, const uint16_t* x, TOut* y, hipStream_t s) {
  const int n = static_cast<int>(w.n), k = static_cast<int>(w.k);
  const int groups = (n + kRowW4 - 1) / kRowW4, per_block = 4 / KS;
  gemv_w4_row_kernel<kRowW4, CH, KS, EXACT, BF, ZP, TOut, false>
      <<<(groups + per_block - 1) / per_block, 256, KS > 1 ? 4 * kRowW4 * sizeof(float) : 0, s>>>(
          static_cast<const uint8_t*>(w.codes), static_cast<const uint16_t*>(w.scales),
          static_cast<const uint8_t*>(w.zeros), x, nullptr, n, k, y);
}

// Act order at M = 1: x in its original column order and the permutation go
// to the kernel, which gathers in LDS (2 * K halfwords).
template <int CH, bool EXACT, bool BF, bool ZP, typename TOut>
void w4_row_perm_go(const bpw_weights& w, const uint16_t* x, TOut* y, hipStream_t s) {
  const int n = static_cast<int>(w.n), k = static_cast<int>(w.k);
  constexpr int rows = kRowW4Perm * kRowW4PermWaves;
  gemv_w4_row_kernel<kRowW4Perm, CH, 1, EXACT, BF, ZP, TOut, true>
      <<<(n + rows - 1) / rows, 64 * kRowW4PermWaves, 4ull * k, s>>>(
          static_cast<const uint8_t*>(w.codes), static_cast<const uint16_t*>(w.scales),
          static_cast<const uint8_t*>(w.zeros), x, w.perm, n, k, y);
}

template <bool BF, bool ZP, typename TOut>
hipError_t w4_perm_dispatch_f(const bpw_weights& w, const uint16_t* x, int m, TOut* y, hipStream_t s) {
  if (m > 1) return w4_skinny<BF, ZP, true>(w, x, m, y, s);
#define BPW_W4RP(E_)                                                    \
  switch ((w.k + 1023) / 1024) {                                        \
    case 1: w4_row_perm_go<1, E_, BF, ZP>(w, x, y, s); break;           \
    case 2: w4_row_perm_go<2, E_, BF, ZP>(w, x, y, s); break;           \
    case 3: w4_row_perm_go<3, E_, BF, ZP>(w, x, y, s); break;           \
    case 4: w4_row_perm_go<4, E_, BF, ZP>(w, x, y, s); break;           \
    case 5: w4_row_perm_go<5, E_, BF, ZP>(w, x, y, s); break;           \
    case 6: w4_row_perm_go<6, E_, BF, ZP>(w, x, y, s); break;           \
    case 7: w4_row_perm_go<7, E_, BF, ZP>(w, x, y, s); break;           \
    default: w4_row_perm_go<8, E_, BF, ZP>(w, x, y, s); break;          \
  }
  if (w.k % 1024 == 0) {
    BPW_W4RP(true)
  } else {
    BPW_W4RP(false)
  }
#undef BPW_W4RP
  return hipGetLastError();
}

template <bool BF, bool ZP, typename TOut>
hipError_t w4_dispatch_f(const bpw_weights& w, const uint16_t* x, int m, TOut* y, float* part, hipStream_t s) {
  if (w4_row_ok(m, w.k)) {
    const int ks = w4_row_split(w.k), ch = w4_row_chunks(w.k);
    const bool exact = w.k == static_cast<int64_t>(ks) * ch * 1024;
    // a split K has 5..8 chunks per wave (9..16 chunks over 2 waves, 17..32 over 4)
#define BPW_W4R1(E_)                                                    \
  switch (ch) {                                                         \
    case 1: w4_row_go<1, 1, E_, BF, ZP>(w, x, y, s); break;             \
    case 2: w4_row_go<2, 1, E_, BF, ZP>(w, x, y, s); break;             \
    case 3: w4_row_go<3, 1, E_, BF, ZP>(w, x, y, s); break;             \
    case 4: w4_row_go<4, 1, E_, BF, ZP>(w, x, y, s); break;             \
    case 5: w4_row_go<5, 1, E_, BF, ZP>(w, x, y, s); break;             \
    case 6: w4_row_go<6, 1, E_, BF, ZP>(w, x, y, s); break;             \
    case 7: w4_row_go<7, 1, E_, BF, ZP>(w, x, y, s); break;             \
    default: w4_row_go<8, 1, E_, BF, ZP>(w, x, y, s); break;            \
  }
#define BPW_W4RS(KS_, E_)                                               \
  switch (ch) {                                                         \
    case 5: w4_row_go<5, KS_, E_, BF, ZP>(w, x, y, s); break;           \
    case 6: w4_row_go<6, KS_, E_, BF, ZP>(w, x, y, s); break;           \
    case 7: w4_row_go<7, KS_, E_, BF, ZP>(w, x, y, s); break;           \
    case 8: w4_row_go<8, KS_, E_, BF, ZP>(w, x, y, s); break;           \
    default: return hipErrorInvalidValue;                               \
  }
    if (ks == 1) {
      if (exact) { BPW_W4R1(true) } else { BPW_W4R1(false) }
    } else if (ks == 2) {
      if (exact) { BPW_W4RS(2, true) } else { BPW_W4RS(2, false) }
    } else {
      if (exact) { BPW_W4RS(4, true) } else { BPW_W4RS(4, false) }
    }
#undef BPW_W4R1
#undef BPW_W4RS
    return hipGetLastError();
  }
  if (w4_skinny_ok(m, w.k)) return w4_skinny<BF, ZP, false>(w, x, m, y, s);
  if (w4_split_ok(m, w.k)) return part ? w4_split<BF, ZP>(w, x, m, y, part, s) : hipErrorInvalidValue;
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
hipError_t w4_dispatch(const bpw_weights& w, const uint16_t* x, bool bf, int m, TOut* y, float* part,
                       hipStream_t s) {
  const bool zp = w.fmt == BPW_INT4_ZP;
  if (bf) return zp ? w4_dispatch_f<true, true>(w, x, m, y, part, s) : w4_dispatch_f<true, false>(w, x, m, y, part, s);
  return zp ? w4_dispatch_f<false, true>(w, x, m, y, part, s) : w4_dispatch_f<false, false>(w, x, m, y, part, s);
}

}  // namespace

bool gemv_t2_fits(int64_t m, int64_t k) { return m >= 1 && m <= 32; }

bool gemv_t2_fused_fits(int64_t m, int64_t k) { return t2_row_ok(m, k); }

hipError_t launch_gemv_t2_fused(const bpw_weights& w, const void* x, int x_dtype, void* y, int y_dtype,
                                hipStream_t s) {
  switch (y_dtype) {
    case BPW_F32: return t2_fused_dispatch(w, x, x_dtype, static_cast<float*>(y), s);
    case BPW_F16: return t2_fused_dispatch(w, x, x_dtype, static_cast<__half*>(y), s);
    default: return t2_fused_dispatch(w, x, x_dtype, static_cast<uint16_t*>(y), s);
  }
}

bool gemv_w4_fits(int64_t m, int64_t k) {
  return m >= 1 && m <= 32 &&
         (w4_row_ok(m, k) || w4_skinny_ok(m, k) || w4_split_ok(m, k) || static_cast<size_t>(m) * k * 2 <= kLdsBudget);
}

size_t gemv_w4_split_bytes(int64_t m, int64_t n, int64_t k) {
  if (!w4_split_ok(m, k)) return 0;
  return static_cast<size_t>(w4_splits(k)) * static_cast<size_t>(m) * static_cast<size_t>(n) * sizeof(float);
}

bool gemv_t2_group_fits(int64_t m, int64_t k) { return m >= 1 && m <= 32; }

size_t gemv_t2_split_bytes(int64_t m, int64_t n, int64_t k, bool group_scales) {
  if (group_scales || !t2_split_ok(m, k)) return 0;
  return static_cast<size_t>(t2_splits(k)) * static_cast<size_t>(m) * static_cast<size_t>(n) * sizeof(float);
}

hipError_t launch_gemv_t2(const bpw_weights& w, const int8_t* q, const float* x_scale, int64_t m,
                          void* y, int y_dtype, bool group_scales, void* ws, size_t ws_bytes, hipStream_t s) {
  const int mi = static_cast<int>(m);
  const size_t need = gemv_t2_split_bytes(m, w.n, w.k, group_scales);
  float* part = need > 0 && ws && ws_bytes >= need ? static_cast<float*>(ws) : nullptr;
  switch (y_dtype) {
    case BPW_F32: return t2_dispatch(w, q, x_scale, mi, static_cast<float*>(y), group_scales, part, s);
    case BPW_F16: return t2_dispatch(w, q, x_scale, mi, static_cast<__half*>(y), group_scales, part, s);
    default: return t2_dispatch(w, q, x_scale, mi, static_cast<uint16_t*>(y), group_scales, part, s);
  }
}

hipError_t launch_gemv_t2_partials(const bpw_weights& w, const int8_t* q, int64_t m, int64_t m0,
                                   int64_t m1, int64_t n0, int64_t n1, int32_t* out,
                                   hipStream_t s) {
  const int k = static_cast<int>(w.k);
  const int mi = static_cast<int>(m);
  if (t2_row_ok(m, k))   // the product for M = 1 runs the row kernel: verify that core
    return t2_row<float, true>(w, q, nullptr, nullptr, out, static_cast<int>(n0), static_cast<int>(n1), s);
  if (t2_stage_ok(m, k, q, w.codes, nullptr, false))   // the staged kernel where the product runs it
    return t2_stage<float, true, false>(w, q, nullptr, mi, static_cast<float*>(nullptr), out, static_cast<int>(m0),
                                        static_cast<int>(m1), static_cast<int>(n0), static_cast<int>(n1), s);
  if (t2_skinny_ok(m, k))   // the skinny kernel for 2 <= M <= 32 up to 32 groups
    return t2_skinny<float, true>(w, q, nullptr, mi, static_cast<float*>(nullptr), out, static_cast<int>(m0),
                                  static_cast<int>(m1), static_cast<int>(n0), static_cast<int>(n1), s);
  if (t2_long_ok(m, k))     // and the long-K kernel for the rest
    return t2_long<float, true>(w, q, nullptr, mi, static_cast<float*>(nullptr), out, static_cast<int>(m0),
                                static_cast<int>(m1), static_cast<int>(n0), static_cast<int>(n1), s);
  return hipErrorInvalidValue;
}

bool gemv_w4_perm_fits(const bpw_weights& w, int64_t m, const void* x) {
  return w.perm != nullptr && (w4_row_perm_ok(m, w.k) || w4_skinny_perm_ok(m, w.k)) &&
         reinterpret_cast<uintptr_t>(x) % 16 == 0 && reinterpret_cast<uintptr_t>(w.perm) % 16 == 0;
}

hipError_t launch_gemv_w4_perm(const bpw_weights& w, const void* x, int x_dtype, int64_t m, void* y,
                               int y_dtype, hipStream_t s) {
  const uint16_t* xh = static_cast<const uint16_t*>(x);
  const bool bf = x_dtype == BPW_BF16, zp = w.fmt == BPW_INT4_ZP;
  const int mi = static_cast<int>(m);
#define BPW_W4P(TOut_)                                                                                   \
  {                                                                                                      \
    TOut_* yo = static_cast<TOut_*>(y);                                                                  \
    if (bf) return zp ? w4_perm_dispatch_f<true, true>(w, xh, mi, yo, s) : w4_perm_dispatch_f<true, false>(w, xh, mi, yo, s); \
    return zp ? w4_perm_dispatch_f<false, true>(w, xh, mi, yo, s) : w4_perm_dispatch_f<false, false>(w, xh, mi, yo, s);       \
  }
  switch (y_dtype) {
    case BPW_F32: BPW_W4P(float)
    case BPW_F16: BPW_W4P(__half)
    default: BPW_W4P(uint16_t)
  }
#undef BPW_W4P
}

hipError_t launch_gemv_w4(const bpw_weights& w, const void* x_sorted, int x_dtype, int64_t m,
                          void* y, int y_dtype, float* part, hipStream_t s) {
  const uint16_t* x = static_cast<const uint16_t*>(x_sorted);
  const bool bf = x_dtype == BPW_BF16;
  const int mi = static_cast<int>(m);
  switch (y_dtype) {
    case BPW_F32: return w4_dispatch(w, x, bf, mi, static_cast<float*>(y), part, s);
    case BPW_F16: return w4_dispatch(w, x, bf, mi, static_cast<__half*>(y), part, s);
    default: return w4_dispatch(w, x, bf, mi, static_cast<uint16_t*>(y), part, s);
  }
}

}  // namespace bpw
