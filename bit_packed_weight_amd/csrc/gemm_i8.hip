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
// Workgroup tile 128 (tokens) x 256 (weight rows), 4 waves; wave w owns weight
// rows [64w, 64w + 64) of the tile and all 128 tokens: 4 x 2 output tiles of
// 32 x 32, i.e. eight "chains" of four MFMAs (one per code plane) per 128-group.
// The fold of one chain (16 conversions + 16 fmas per lane) runs while the next
// chain's MFMAs execute, so the VALU and the matrix core work side by side.
//
// Activations (plane order, 128 bytes per row and group) stream global -> LDS
// by direct loads into a double buffer; each wave reads its A operands from LDS
// one 32-row tile ahead. Weights never touch LDS: each lane loads its own 16
// code bytes per 32-row weight tile and group one group ahead and decodes them
// straight into B operands.
//
// The same kernel takes 4-bit weights ("TensorFold PR #1176", the int8 prompt
// GEMM: an affine 4-bit code is an exact int8, so the group dot runs on the
// int8 matrix core). Each lane then loads 32 code bytes per weight tile and
// group and decodes every nibble to the signed byte code - zero, so the int32
// MFMA result is again the exact partial P[m,n,g] = sum q * (code - zero) and
// the fold is unchanged (symmetric codes, zero 8, decode to 16 (code - 8) in
// fewer instructions; their chains carry 16 P and fold with scale / 16). The activations
// come in nibble order: within each 8 bytes of a row, the even-indexed
// elements, then the odd ones, in the chunk arrangement of the plane order.
// For K a multiple of 1024 the 4-bit codes do pass through LDS: direct copies
// issued three groups ahead, so that their HBM latency leaves the loop.
#include "device.h"
#include "lds_dma.h"
#include "launch.h"
#include "store.h"

namespace bpw {
namespace {

constexpr int BM = 128, BN = 256, NT = 256;
constexpr int A_ROW = 128;                      // one 128-group of a row, plane order
constexpr int A_BYTES = BM * A_ROW;             // one LDS buffer (16 KB)
constexpr int LDS_BYTES = 2 * A_BYTES;
constexpr int GROUP_M = 4;                      // tile raster: 4 token tiles per column sweep
// Codes-ahead 4-bit form: after the A buffers, three code slots (4 waves x 64
// rows x 64 bytes each), then the scale rows (BN x G fp16) and zero-point rows
// (BN x G / 2 bytes).
constexpr int DEEP_NS = 3;
constexpr int DEEP_SLOT = 4 * 64 * 64;
constexpr int DEEP_OC = LDS_BYTES;
constexpr int DEEP_OS = DEEP_OC + DEEP_NS * DEEP_SLOT;
constexpr int deep_lds(int g, bool zp) { return DEEP_OS + 2 * BN * g + (zp ? BN * (g >> 1) : 0); }

__device__ __forceinline__ int d_row(int r, int h) { return 8 * (r >> 2) + 4 * h + (r & 3); }

template <int V>
struct IntC {
  static constexpr int value = V;
};

// 16-byte LDS read straight into AGPRs (the MFMA reads its A operand from
// there), leaving the VGPRs to the accumulators, group partials and B
// operands. The compiler does not track this read: ds_wait_agpr must run
// before the registers are used.
template <int OFF>
__device__ __forceinline__ void ds_read_agpr(v4i& dst, uint32_t addr) {
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=a"(dst) : "v"(addr), "i"(OFF));
}
// Wait for every outstanding LDS read; the operands are tied to the wait so
// that no use of them can be scheduled before it.
__device__ __forceinline__ void ds_wait_agpr(v4i (&a)[4]) {
  asm volatile("s_waitcnt lgkmcnt(0)" : "+a"(a[0]), "+a"(a[1]), "+a"(a[2]), "+a"(a[3]));
}

// Logical tile -> (token tile, weight tile): runs of GROUP_M token tiles sweep
// the weight tiles, so workgroups that run together share activation and code
// slices in L2.
__device__ __forceinline__ void tile_coords(int t, int mtiles, int ntiles, int& mt, int& nt) {
  const int per = GROUP_M * ntiles;
  const int first = (t / per) * GROUP_M;
  const int gs = min(mtiles - first, GROUP_M);
  const int r = t % per;
  mt = first + r % gs;
  nt = r / gs;
}

// Weight formats of the kernel: ternary codes, 4-bit symmetric (zero 8), 4-bit
// with a zero point per (row, group).
enum { WF_T2 = 0, WF_I4 = 1, WF_I4Z = 2 };

template <typename TOut, bool PARTIALS, int WF, bool DEEP = false>
__global__ __launch_bounds__(NT, 1) void gemm_t2_kernel(
    const int8_t* __restrict__ qp, const float* __restrict__ x_scale,
    const uint8_t* __restrict__ codes, const uint16_t* __restrict__ wscale,
    const uint8_t* __restrict__ zeros, int bf_scale, int M, int N, int K,
    TOut* __restrict__ y, int32_t* __restrict__ pout, int pm0, int pm1, int pn0, int pn1,
    int mt0, int mtiles, int nt0, int ntiles) {
  extern __shared__ __align__(16) uint8_t smem[];
  constexpr bool W4 = WF != WF_T2;
  const int G = K >> 7;
  const int KB = W4 ? (K >> 1) : (K >> 2);
  const int ZB = (G + 1) >> 1;
  const bool bfs = W4 && bf_scale;
  // Fold scale of a group; symmetric 4-bit chains carry 16 P (see decode).
  auto scale_f32 = [&](uint16_t bits) __attribute__((always_inline)) {
    const float v = bfs ? bf16_to_f32(bits) : __half2float(__builtin_bit_cast(__half, bits));
    return WF == WF_I4 ? v * 0.0625f : v;
  };
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int mt, nt;
  tile_coords(xcd_swizzle(blockIdx.x, mtiles * ntiles), mtiles, ntiles, mt, nt);
  mt += mt0;
  nt += nt0;
  const int m0 = mt * BM, n0 = nt * BN;
  const int n = lane & 31, h = lane >> 5;

  // A: row r of a buffer is 8 chunks of 16 bytes; chunk c sits in slot
  // c ^ ((r >> 1) & 7). Two 128-byte rows share one pass over the 64 LDS banks,
  // so the 16 rows a 16-lane phase of one MFMA read touches (8 even, 8 odd)
  // land on 16 distinct bank groups.
  // Direct load t (0..3) of wave w fills LDS bytes [(4w + t) * 1024, +1024):
  // rows 8 (4w + t) + lane / 8, slot lane % 8; ((row >> 1) & 7) is
  // (4t + lane / 16) & 7.
  const int a_row0 = 32 * wave + (lane >> 3);
  // (4t + lane / 16) & 7 takes two values: t even, t odd.
  const int8_t* a_base[2] = {qp + 16 * ((lane & 7) ^ ((lane >> 4) & 7)),
                             qp + 16 * ((lane & 7) ^ ((4 + (lane >> 4)) & 7))};
  int a_row[4];                                      // token rows past the end are clamped
#pragma unroll
  for (int t = 0; t < 4; ++t) a_row[t] = min(m0 + a_row0 + 8 * t, M - 1);
  const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<size_t>(smem)) + wave * 4096;
  auto a_load = [&](int g, int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int8_t* src = a_base[t & 1] + static_cast<size_t>(a_row[t]) * K + g * 128;
      lds_dma16(src, __builtin_amdgcn_readfirstlane(lds0 + buf * A_BYTES + t * 1024));
    }
  };
  // A operand reads (into AGPRs, see ds_read_agpr): plane t of token row
  // 32 i + n is chunk 2t + h; the buffer and token tile are immediate offsets
  // (32 i rows shift (row >> 1) by 16 i: the slot does not depend on i).
  uint32_t a_addr[4];
#pragma unroll
  for (int t = 0; t < 4; ++t)
    a_addr[t] = static_cast<uint32_t>(reinterpret_cast<size_t>(smem)) + n * A_ROW + 16 * ((2 * t + h) ^ ((n >> 1) & 7));
  auto a_read = [&](auto BUFC, auto IC, v4i (&dst)[4]) __attribute__((always_inline)) {
    constexpr int OFF = decltype(BUFC)::value * A_BYTES + decltype(IC)::value * 32 * A_ROW;
#pragma unroll
    for (int t = 0; t < 4; ++t) ds_read_agpr<OFF>(dst[t], a_addr[t]);
  };

  // B: this lane's two weight rows (one per 32-row tile of the wave). Lane
  // half h takes weights [64h, 64h + 64) of each group: 16 ternary or 32
  // 4-bit code bytes.
  const uint8_t* b_src[2];
  const uint16_t* s_src[2];
  const uint8_t* z_src[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const size_t row = static_cast<size_t>(min(n0 + 64 * wave + 32 * j + n, N - 1));
    b_src[j] = codes + row * KB + (W4 ? 32 : 16) * h;
    s_src[j] = wscale + row * G;
    z_src[j] = WF == WF_I4Z ? zeros + row * ZB : nullptr;
  }
  // Raw bytes only (the scale is converted a group later, so that nothing
  // waits on these loads before it has to).
  struct Raw {
    v4u c[2][W4 ? 2 : 1];
    uint16_t s[2];
    uint32_t z[2];        // zero-point byte of the row (two groups), and the group's nibble shift
    uint32_t zsh;
  };
  auto raw_load = [&](Raw& r, int g) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      if (W4) {
        r.c[j][0] = *reinterpret_cast<const v4u*>(b_src[j] + g * 64);
        r.c[j][W4 ? 1 : 0] = *reinterpret_cast<const v4u*>(b_src[j] + g * 64 + 16);
      } else {
        r.c[j][0] = *reinterpret_cast<const v4u*>(b_src[j] + g * 32);
      }
      r.s[j] = s_src[j][g];
      r.z[j] = WF == WF_I4Z ? static_cast<uint32_t>(z_src[j][g >> 1]) : 0u;
    }
    r.zsh = 4u * static_cast<uint32_t>(g & 1);
  };
  // Codes-ahead form of the 4-bit weights (DEEP): each wave copies its 64
  // code rows of a group (64 x 64 bytes, four 1 KB direct copies) into one of
  // three LDS slots, at the top of the group three before it, and the
  // workgroup's scale (and zero-point) rows for all groups are staged once.
  // The loop then holds no compiler-tracked global load, so its waits count
  // only these copies, and the next group's raw weights come from LDS. The
  // wait at the end of each group, for the next group's activations, covers
  // every older copy too: group g + 2's codes, issued a group earlier. Row r
  // of a wave's slot keeps its four 16-byte units at r * 64 + 16 (u ^ ((r >>
  // 2) & 3)): the 16 rows that one quarter-wave reads then cover all 64 banks.
  // (Measured at M=2048, K=4096, N=14336, symmetric codes: 196 -> 189-190 us
  // per call, then 182 us with the LDS read placed as below; two slots, with a
  // wait for the next group's codes in the middle of each group, 192-193 us.)
  const int G8 = G >> 3;                                   // DEEP: K % 1024 == 0
  const uint32_t lds_code = static_cast<uint32_t>(reinterpret_cast<size_t>(smem)) + DEEP_OC + wave * 4096;
  auto code_copy = [&](int g, int slot) __attribute__((always_inline)) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int r = 16 * k + (lane >> 2);
      const int u = (lane & 3) ^ ((r >> 2) & 3);
      const size_t row = static_cast<size_t>(min(n0 + 64 * wave + r, N - 1));
      lds_dma16(codes + row * KB + g * 64 + 16 * u,
                __builtin_amdgcn_readfirstlane(lds_code + slot * DEEP_SLOT + k * 1024));
    }
  };
  auto lds_raw = [&](Raw& r, int g, int slot) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int rr = 32 * j + n;
      const uint8_t* base = smem + DEEP_OC + slot * DEEP_SLOT + wave * 4096 + rr * 64;
      r.c[j][0] = *reinterpret_cast<const v4u*>(base + 16 * ((2 * h) ^ ((rr >> 2) & 3)));
      r.c[j][W4 ? 1 : 0] = *reinterpret_cast<const v4u*>(base + 16 * ((2 * h + 1) ^ ((rr >> 2) & 3)));
      const int R = 64 * wave + rr;
      r.s[j] = reinterpret_cast<const uint16_t*>(smem + DEEP_OS)[R * G + g];
      r.z[j] = WF == WF_I4Z ? static_cast<uint32_t>(smem[DEEP_OS + 2 * BN * G + R * (G >> 1) + (g >> 1)]) : 0u;
    }
    r.zsh = 4u * static_cast<uint32_t>(g & 1);
  };
  // Ternary: 16 code bytes -> the four code planes as signed MFMA B operands.
  // Lane half h, plane t, byte 4q + p holds the weight at 64h + 16q + 4p + t
  // of the group, matching plane-ordered activations at offset 32t + 16h + 4q + p.
  // 4-bit: 32 code bytes (dwords d0..d7) -> MFMA t takes dwords 2t and 2t + 1
  // as (low nibbles, high nibbles) of each, so byte 4q + p holds the weight at
  // 64h + 16t + 8(q >> 1) + 2p + (q & 1), matching nibble-ordered activations
  // at the same offset 32t + 16h + 4q + p.
  auto decode = [&](const Raw& r, int j, v4i (&b)[4]) __attribute__((always_inline)) {
    if (WF == WF_I4) {
      // Symmetric codes: w ^ 0x88888888 holds code - 8 as a 4-bit two's
      // complement in every nibble; moved to the top of its byte it is the
      // signed byte 16 (code - 8). The chain result is then exactly 16 P
      // (|16 P| < 2^22), and the fold takes scale / 16 (exact).
      const uint32_t d[8] = {r.c[j][0].x, r.c[j][0].y, r.c[j][0].z, r.c[j][0].w,
                             r.c[j][W4 ? 1 : 0].x, r.c[j][W4 ? 1 : 0].y, r.c[j][W4 ? 1 : 0].z, r.c[j][W4 ? 1 : 0].w};
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const uint32_t e0 = d[2 * t] ^ 0x88888888u, e1 = d[2 * t + 1] ^ 0x88888888u;
        b[t] = v4i{static_cast<int>((e0 << 4) & 0xF0F0F0F0u), static_cast<int>(e0 & 0xF0F0F0F0u),
                   static_cast<int>((e1 << 4) & 0xF0F0F0F0u), static_cast<int>(e1 & 0xF0F0F0F0u)};
      }
    } else if (W4) {
      const uint32_t z = WF == WF_I4Z ? ((r.z[j] >> r.zsh) & 15u) : 8u;
      const uint32_t zadd = (0x80u - z) * 0x01010101u;
      const uint32_t d[8] = {r.c[j][0].x, r.c[j][0].y, r.c[j][0].z, r.c[j][0].w,
                             r.c[j][W4 ? 1 : 0].x, r.c[j][W4 ? 1 : 0].y, r.c[j][W4 ? 1 : 0].z, r.c[j][W4 ? 1 : 0].w};
#pragma unroll
      for (int t = 0; t < 4; ++t)
        b[t] = v4i{static_cast<int>(nib_lo_signed(d[2 * t], zadd)), static_cast<int>(nib_hi_signed(d[2 * t], zadd)),
                   static_cast<int>(nib_lo_signed(d[2 * t + 1], zadd)),
                   static_cast<int>(nib_hi_signed(d[2 * t + 1], zadd))};
    } else {
      const v4u& c = r.c[j][0];
#pragma unroll
      for (int t = 0; t < 4; ++t)
        b[t] = v4i{static_cast<int>(code_plane_signed(c.x, t)), static_cast<int>(code_plane_signed(c.y, t)),
                   static_cast<int>(code_plane_signed(c.z, t)), static_cast<int>(code_plane_signed(c.w, t))};
    }
  };

  v16f acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = v16f{};

  // Fold (or, for the partials entry, store) the int32 result of chain (i, j)
  // of group g.
  auto fold = [&](const v16i& d, int i, int j, float s, int g) __attribute__((always_inline)) {
    if (PARTIALS) {
      const int nn = n0 + 64 * wave + 32 * j + n;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int mm = m0 + 32 * i + d_row(r, h);
        if (mm >= pm0 && mm < pm1 && nn >= pn0 && nn < pn1)
          pout[(static_cast<size_t>(mm - pm0) * (pn1 - pn0) + (nn - pn0)) * G + g] = WF == WF_I4 ? (d[r] >> 4) : d[r];
      }
    } else {
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = fmaf(static_cast<float>(d[r]), s, acc[i][j][r]);
    }
  };
  auto chain = [&](const v4i (&a)[4], const v4i (&b)[4]) __attribute__((always_inline)) {
    v16i d = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[0], b[0], v16i{}, 0, 0, 0);
#pragma unroll
    for (int t = 1; t < 4; ++t) d = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[t], b[t], d, 0, 0, 0);
    return d;
  };

  v4i aop[2][4];        // A operands (AGPRs) of the current and next 32-row token tile
  v4i bop[2][4];        // B operands of the wave's two weight tiles
  v16i dprev = {};      // the chain whose fold is pending (none before group 0)
  float sprev = 0.0f;
  Raw raw;

  if constexpr (DEEP) {
    // the workgroup's scale rows (BN x G fp16, contiguous in the plane; rows
    // past N repeat the last valid 16-byte piece, never read) and zero-point
    // rows (BN x G / 2 bytes, 4-byte pieces), wave w taking every fourth copy
    const int rows = min(BN, N - n0);
    const uint8_t* sp = reinterpret_cast<const uint8_t*>(wscale) + static_cast<size_t>(n0) * G * 2;
    const int slast = rows * G8 - 1;                       // last valid 16-byte piece
    for (int c = wave; c < 4 * G8; c += 4)                  // 32 G pieces, 64 per copy
      lds_dma16(sp + 16 * min(64 * c + lane, slast),
                __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(reinterpret_cast<size_t>(smem)) + DEEP_OS +
                                               c * 1024));
    if (WF == WF_I4Z) {
      const uint8_t* zp = zeros + static_cast<size_t>(n0) * (G >> 1);
      const int zlast = rows * G8 - 1;                       // last valid 4-byte piece
      for (int c = wave; c < 4 * G8; c += 4)                // 32 G pieces, 64 per copy
        lds_dma4(zp + 4 * min(64 * c + lane, zlast),
                 __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(reinterpret_cast<size_t>(smem)) + DEEP_OS +
                                                2 * BN * G + c * 256));
    }
    a_load(0, 0);
#pragma unroll
    for (int c = 0; c < DEEP_NS; ++c) code_copy(min(c, G - 1), c);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    lds_raw(raw, 0, 0);
  } else {
    a_load(0, 0);
    raw_load(raw, 0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }
  decode(raw, 0, bop[0]);
  float s0 = scale_f32(raw.s[0]), s1 = scale_f32(raw.s[1]);

  // One 128-group in LDS buffer BUF. On entry: bop[0] holds this group's first
  // weight tile, raw its raw bytes, dprev/sprev the previous group's last chain
  // (zero before group 0). An AGPR read is always waited for inside the same
  // group, so no register copy of a value still in flight can be placed at the
  // loop edge. The
  // body has no branches: after the last group the loads and decodes of
  // "group g + 1" repeat the last group and are not used.
  auto group = [&](int g, auto BUFC) __attribute__((always_inline)) {
    constexpr int BUF = decltype(BUFC)::value;
    const int gn = min(g + 1, G - 1);
    // The next group's raw weights: 4-bit codes (32 bytes a lane) go out first
    // in the group, ternary codes after the first chain (measured: 4-bit at
    // M=2048, K=4096, N=14336 200.6 -> 195.4 us; ternary at M=4096, K=8192,
    // N=28672 1148 -> 1199 us if moved too).
    Raw nraw;
    if (W4 && !DEEP) {
      raw_load(nraw, gn);
      __builtin_amdgcn_sched_barrier(0);
    }
    a_read(IntC<BUF>{}, IntC<0>{}, aop[0]);
    // The other buffer was last read before the previous barrier.
    a_load(gn, BUF ^ 1);
    // DEEP: group g + 3's codes into the slot group g's codes left (read into
    // registers during group g - 1)
    if (DEEP) code_copy(min(g + DEEP_NS, G - 1), g % DEEP_NS);
    if (!PARTIALS || g > 0) fold(dprev, 3, 1, sprev, g - 1);
    ds_wait_agpr(aop[0]);
    __builtin_amdgcn_sched_barrier(0);
    // chain (0,0); decode this group's second weight tile; read token tile 1.
    {
      const v16i d = chain(aop[0], bop[0]);
      decode(raw, 1, bop[1]);
      a_read(IntC<BUF>{}, IntC<1>{}, aop[1]);
      dprev = d;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 11, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if (!W4) {
      raw_load(nraw, gn);
      __builtin_amdgcn_sched_barrier(0);
    }
    // Chains (0,1) (1,0) (1,1) ... (3,1); each folds its predecessor. Token
    // tile i + 1 is read during chain (i, 0), into the registers that chain
    // (i - 1, 1) used, and waited for before chain (i + 1, 0).
    auto slot = [&](auto CC) __attribute__((always_inline)) {
      constexpr int c = decltype(CC)::value, i = c >> 1, j = c & 1;
      if (j == 0) ds_wait_agpr(aop[i & 1]);
      const v16i d = chain(aop[i & 1], bop[j]);
      constexpr int pi = (c - 1) >> 1, pj = (c - 1) & 1;
      fold(dprev, pi, pj, pj ? s1 : s0, g);
      if (j == 0 && i < 3) a_read(IntC<BUF>{}, IntC<i + 1>{}, aop[(i + 1) & 1]);
      if (DEEP && c == 6) {
        // (read during chain (3,0): measured at M=2048, K=4096, N=14336,
        // 181.6-182.8 us; during chain (1,1), (2,1) or (3,1), 187-189 us)
        // group g + 1's codes landed before the end of group g - 1 (PARTIALS
        // stores in fold, and stores count in vmcnt too: that path waits for
        // every copy here and at the end of the group)
        if (PARTIALS) wait_vmcnt<0>();
        asm volatile("" ::: "memory");
        lds_raw(nraw, gn, (g + 1) % DEEP_NS);
      }
      // this group's first weight tile is free after chain (3,0): decode the next one
      if (c == 7) decode(nraw, 0, bop[0]);
      dprev = d;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (c == 7)
          __builtin_amdgcn_sched_group_barrier(0x002, 19, 0);
        else
          __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    };
    slot(IntC<1>{});
    slot(IntC<2>{});
    slot(IntC<3>{});
    slot(IntC<4>{});
    slot(IntC<5>{});
    slot(IntC<6>{});
    slot(IntC<7>{});
    sprev = s1;
    raw = nraw;
    s0 = scale_f32(nraw.s[0]);
    s1 = scale_f32(nraw.s[1]);
    if (DEEP && !PARTIALS) {
      // the direct A loads have landed, and every older copy with them (group
      // g + 2's codes); group g + 3's four code copies may be in flight
      __builtin_amdgcn_sched_barrier(0);
      wait_vmcnt<4>();
      asm volatile("" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
    } else {
      __builtin_amdgcn_s_waitcnt(0);   // the direct A loads and raw weights have landed
    }
    __syncthreads();
  };
  int g = 0;
  for (; g + 1 < G; g += 2) {
    group(g, IntC<0>{});
    group(g + 1, IntC<1>{});
  }
  if (g < G) group(g, IntC<0>{});
  if (DEEP) wait_vmcnt<0>();         // no copy into LDS outlives the loop
  fold(dprev, 3, 1, sprev, G - 1);
  if (PARTIALS) return;

  // Epilogue: each 32 x 64 block of the wave goes through LDS (8 KB per wave,
  // the A buffers are free once every wave is past this barrier) so that the
  // output leaves in row segments of 4 values per lane instead of single
  // 2-byte stores.
  __syncthreads();
  float* stage = reinterpret_cast<float*>(smem + wave * 8192);
  const bool vec = (N & 3) == 0;
  // Row scales of the 32 rows this lane stores, loaded together up front.
  float xsv[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int q = 0; q < 8; ++q) xsv[i][q] = x_scale[min(m0 + 32 * i + 4 * q + (lane >> 4), M - 1)];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
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
        const float xs = xsv[i][q];
        const float v[4] = {__uint_as_float(raw4.x) * xs, __uint_as_float(raw4.y) * xs,
                            __uint_as_float(raw4.z) * xs, __uint_as_float(raw4.w) * xs};
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

// ---------------------------------------------------------------------------
// Per-(token, group) activation scales on the int8 matrix core:
//  * the affine 4-bit x int8 product of "TensorFold PR #1176" ("What changes":
//    per group s * a * (code . q) + b * sum(x), the dot on the raw codes 0..15,
//    with b = -zero * s here), FX_AFF_SYM (zero 8) and FX_AFF_ZP;
//  * ternary weights x int8 with one activation scale per (row, 128-group),
//    FX_T2G ("Kernel experiments", Test 7: acc += partial * x_scale * w_scale).
//
// Same tile as gemm_t2_kernel (128 tokens x 256 weight rows, 4 waves; wave w
// owns weight rows [64w, 64w + 64) and all 128 tokens), but every MFMA takes
// the weights as its first operand, so lane l of a 32 x 32 result holds token
// 32 i + (l & 31) and 16 weight rows: the token's activation scale and sum are
// one value per lane. The weight scales of each group are staged in LDS as
// fp32 by the workgroup (one row per thread) and read 16 at a time, for one
// 32-row weight tile, just before that tile's chains. Chains run weight tile
// by weight tile, (0,0) (1,0) (2,0) (3,0) then (0,1) .. (3,1), over A operands
// of the four token tiles kept in AGPRs (read one tile ahead during the first
// weight tile's chains), so only one tile's scales and B operands are live.
//
// Affine fold: the int32 dot D (|D| <= 127 * 15 * 128 < 2^24) converts to fp32
// exactly; t = fma(D, a, -8 * sum) for symmetric codes (b = -8 s, so s * t is
// the group's term), t = D * a with zero points; then acc += s * t, and with
// zero points acc += b * sum. (The page saves the conversion by starting each
// chain at the bit pattern of 12582912.0f and removing it in the same fma that
// applies a; the rounding of that fma's constant costs up to one unit of D per
// group, an absolute error that broke the 1e-3 parity bound on outputs near
// zero, so the exact form is used.)
// Ternary: acc += s * (float(P) * xs).
enum { FX_T2G = 0, FX_AFF_SYM = 1, FX_AFF_ZP = 2 };
constexpr int LDS_G_SCALE = LDS_BYTES;               // [2][256] fp32 weight scales of a group
constexpr int LDS_G_BIAS = LDS_BYTES + 2048;         // [2][256] fp32 b = -zero * scale (zero points)
constexpr int STAGE_ROW = 68;                        // epilogue stage row (floats): 16-byte aligned, fewer conflicts
constexpr int LDS_G_BYTES = LDS_BYTES + 4096 > 4 * 32 * STAGE_ROW * 4 ? LDS_BYTES + 4096 : 4 * 32 * STAGE_ROW * 4;

// 16-byte LDS read into VGPRs, untracked like ds_read_agpr: ds_wait_v4 must run
// before the registers are used.
template <int OFF>
__device__ __forceinline__ void ds_read_v(v4f& dst, uint32_t addr) {
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(dst) : "v"(addr), "i"(OFF));
}
__device__ __forceinline__ void ds_wait_v4(v4f (&a)[4]) {
  asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]));
}

template <typename TOut, bool PARTIALS, int FX>
__global__ __launch_bounds__(NT, 1) void gemm_g_kernel(
    const int8_t* __restrict__ qp, const float* __restrict__ xsc,
    const uint8_t* __restrict__ codes, const uint16_t* __restrict__ wscale,
    const uint8_t* __restrict__ zeros, int bf_scale, int M, int N, int K,
    TOut* __restrict__ y, int32_t* __restrict__ pout, int pm0, int pm1, int pn0, int pn1,
    int mt0, int mtiles, int nt0, int ntiles) {
  extern __shared__ __align__(16) uint8_t smem[];
  constexpr bool W4 = FX != FX_T2G;
  constexpr bool ZP = FX == FX_AFF_ZP;
  const int G = K >> 7;
  const int KB = W4 ? (K >> 1) : (K >> 2);
  const int ZB = (G + 1) >> 1;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int mt, nt;
  tile_coords(xcd_swizzle(blockIdx.x, mtiles * ntiles), mtiles, ntiles, mt, nt);
  mt += mt0;
  nt += nt0;
  const int m0 = mt * BM, n0 = nt * BN;
  const int n = lane & 31, h = lane >> 5;
  const uint32_t sbase = static_cast<uint32_t>(reinterpret_cast<size_t>(smem));

  // A (activations, plane or nibble order): the same direct loads, swizzle and
  // AGPR reads as gemm_t2_kernel.
  const int a_row0 = 32 * wave + (lane >> 3);
  const int8_t* a_base[2] = {qp + 16 * ((lane & 7) ^ ((lane >> 4) & 7)),
                             qp + 16 * ((lane & 7) ^ ((4 + (lane >> 4)) & 7))};
  int a_row[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) a_row[t] = min(m0 + a_row0 + 8 * t, M - 1);
  const uint32_t lds0 = sbase + wave * 4096;
  auto a_load = [&](int g, int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int8_t* src = a_base[t & 1] + static_cast<size_t>(a_row[t]) * K + g * 128;
      lds_dma16(src, __builtin_amdgcn_readfirstlane(lds0 + buf * A_BYTES + t * 1024));
    }
  };
  uint32_t a_addr[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) a_addr[t] = sbase + n * A_ROW + 16 * ((2 * t + h) ^ ((n >> 1) & 7));
  auto a_read = [&](auto BUFC, auto IC, v4i (&dst)[4]) __attribute__((always_inline)) {
    constexpr int OFF = decltype(BUFC)::value * A_BYTES + decltype(IC)::value * 32 * A_ROW;
#pragma unroll
    for (int t = 0; t < 4; ++t) ds_read_agpr<OFF>(dst[t], a_addr[t]);
  };

  // B (weights): lane row 32 j + n of the wave's 64, as in gemm_t2_kernel.
  const uint8_t* b_src[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const size_t row = static_cast<size_t>(min(n0 + 64 * wave + 32 * j + n, N - 1));
    b_src[j] = codes + row * KB + (W4 ? 32 : 16) * h;
  }
  struct Raw {
    v4u c[2][W4 ? 2 : 1];
  };
  auto raw_load = [&](Raw& r, int g) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      if (W4) {
        r.c[j][0] = *reinterpret_cast<const v4u*>(b_src[j] + g * 64);
        r.c[j][W4 ? 1 : 0] = *reinterpret_cast<const v4u*>(b_src[j] + g * 64 + 16);
      } else {
        r.c[j][0] = *reinterpret_cast<const v4u*>(b_src[j] + g * 32);
      }
    }
  };
  // Raw 4-bit codes (0..15) as MFMA bytes in nibble order (low nibbles of a
  // dword, then its high nibbles), or ternary codes as signed -1/0/1/2 bytes.
  auto decode = [&](const Raw& r, int j, v4i (&b)[4]) __attribute__((always_inline)) {
    if (W4) {
      const uint32_t d[8] = {r.c[j][0].x, r.c[j][0].y, r.c[j][0].z, r.c[j][0].w,
                             r.c[j][W4 ? 1 : 0].x, r.c[j][W4 ? 1 : 0].y, r.c[j][W4 ? 1 : 0].z, r.c[j][W4 ? 1 : 0].w};
#pragma unroll
      for (int t = 0; t < 4; ++t)
        b[t] = v4i{static_cast<int>(d[2 * t] & 0x0F0F0F0Fu), static_cast<int>((d[2 * t] >> 4) & 0x0F0F0F0Fu),
                   static_cast<int>(d[2 * t + 1] & 0x0F0F0F0Fu), static_cast<int>((d[2 * t + 1] >> 4) & 0x0F0F0F0Fu)};
    } else {
      const v4u& c = r.c[j][0];
#pragma unroll
      for (int t = 0; t < 4; ++t)
        b[t] = v4i{static_cast<int>(code_plane_signed(c.x, t)), static_cast<int>(code_plane_signed(c.y, t)),
                   static_cast<int>(code_plane_signed(c.z, t)), static_cast<int>(code_plane_signed(c.w, t))};
    }
  };

  // Weight scale (and zero point) of row n0 + tid, staged per group: raw bits
  // loaded a group ahead, converted and written to LDS at the group's end.
  const size_t srow = static_cast<size_t>(min(n0 + tid, N - 1));
  const uint16_t* s_row = wscale + srow * G;
  const uint8_t* z_row = ZP ? zeros + srow * ZB : nullptr;
  auto stage_scale = [&](uint16_t sbits, uint32_t zbyte, int g, int buf) __attribute__((always_inline)) {
    const float sv = (W4 && bf_scale) ? bf16_to_f32(sbits) : __half2float(__builtin_bit_cast(__half, sbits));
    float* sl = reinterpret_cast<float*>(smem + LDS_G_SCALE + buf * 1024);
    sl[tid] = sv;
    if (ZP) {
      const float z = static_cast<float>((zbyte >> (4 * (g & 1))) & 15u);
      reinterpret_cast<float*>(smem + LDS_G_BIAS + buf * 1024)[tid] = -z * sv;   // exact
    }
  };
  // This lane's weight rows of tile j: 64 wave + 32 j + 8 q + 4 h + p for element
  // 4 q + p of the chain result.
  const uint32_t s_addr = sbase + LDS_G_SCALE + (64 * wave + 4 * h) * 4;
  auto s_read = [&](auto BUFC, auto JC, v4f (&sv)[4], v4f (&bv)[4]) __attribute__((always_inline)) {
    constexpr int OFF = decltype(BUFC)::value * 1024 + decltype(JC)::value * 128;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (q == 0) ds_read_v<OFF>(sv[0], s_addr);
      if (q == 1) ds_read_v<OFF + 32>(sv[1], s_addr);
      if (q == 2) ds_read_v<OFF + 64>(sv[2], s_addr);
      if (q == 3) ds_read_v<OFF + 96>(sv[3], s_addr);
    }
    if (ZP) {
      ds_read_v<OFF + 2048>(bv[0], s_addr);
      ds_read_v<OFF + 2048 + 32>(bv[1], s_addr);
      ds_read_v<OFF + 2048 + 64>(bv[2], s_addr);
      ds_read_v<OFF + 2048 + 96>(bv[3], s_addr);
    }
  };

  // Token values of this lane (token 32 i + n of the tile), loaded a group ahead:
  // affine (a, sum) pairs of [M][G][2], ternary scales of [M][G].
  const float* tok_src[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const size_t mm = static_cast<size_t>(min(m0 + 32 * i + n, M - 1));
    tok_src[i] = PARTIALS ? nullptr : xsc + mm * G * (W4 ? 2 : 1);
  }
  struct Tok {
    float a[4], x[4];
  };
  auto tok_load = [&](Tok& t, int g) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (PARTIALS) {                    // the partials entry has no token values (xsc is NULL)
        t.a[i] = t.x[i] = 0.0f;
        continue;
      }
      if (W4) {
        const float2 v = *reinterpret_cast<const float2*>(tok_src[i] + 2 * g);
        t.a[i] = v.x;
        t.x[i] = v.y;
      } else {
        t.a[i] = tok_src[i][g];
        t.x[i] = 0.0f;
      }
    }
  };
  // Per-lane fold constants of a group: av (a or xs), cv (the fma constant), sx (sum).
  float av[4], cv[4], sx[4];
  auto tok_set = [&](const Tok& t) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      av[i] = t.a[i];
      sx[i] = t.x[i];
      cv[i] = FX == FX_AFF_SYM ? -8.0f * t.x[i] : 0.0f;     // exact
    }
  };

  v16f acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = v16f{};

  v4f sv[4], bv[4];       // the current weight tile's scales (and b) for elements 4q + p
#pragma unroll
  for (int q = 0; q < 4; ++q) sv[q] = bv[q] = v4f{};
  // Fold (or, for the partials entry, store) chain (i, j) of group g.
  auto fold = [&](const v16i& d, int i, int j, int g) __attribute__((always_inline)) {
    if (PARTIALS) {
      const int mm = m0 + 32 * i + n;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int nn = n0 + 64 * wave + 32 * j + d_row(r, h);
        if (mm >= pm0 && mm < pm1 && nn >= pn0 && nn < pn1)
          pout[(static_cast<size_t>(mm - pm0) * (pn1 - pn0) + (nn - pn0)) * G + g] = d[r];
      }
    } else {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float s1 = sv[r >> 2][r & 3];
        if (W4) {
          const float t = fmaf(static_cast<float>(d[r]), av[i], cv[i]);
          acc[i][j][r] = fmaf(t, s1, acc[i][j][r]);
          if (ZP) acc[i][j][r] = fmaf(bv[r >> 2][r & 3], sx[i], acc[i][j][r]);
        } else {
          acc[i][j][r] = fmaf(static_cast<float>(d[r]) * av[i], s1, acc[i][j][r]);
        }
      }
    }
  };
  auto chain = [&](const v4i (&b)[4], const v4i (&a)[4]) __attribute__((always_inline)) {
    v16i d = __builtin_amdgcn_mfma_i32_32x32x32_i8(b[0], a[0], v16i{}, 0, 0, 0);
#pragma unroll
    for (int t = 1; t < 4; ++t) d = __builtin_amdgcn_mfma_i32_32x32x32_i8(b[t], a[t], d, 0, 0, 0);
    return d;
  };

  v4i aop[4][4];          // A operands (AGPRs) of the four token tiles
  v4i bop[4];             // B operands of the weight tile in use
  v16i dprev = {};        // the chain whose fold is pending
  Raw raw;
  Tok tok;

  // Prologue: group 0's activations, codes, token values and staged scales.
  a_load(0, 0);
  raw_load(raw, 0);
  tok_load(tok, 0);
  {
    const uint16_t sb = s_row[0];
    const uint32_t zb = ZP ? static_cast<uint32_t>(z_row[0]) : 0u;
    __builtin_amdgcn_s_waitcnt(0);
    stage_scale(sb, zb, 0, 0);
  }
  __syncthreads();
  decode(raw, 0, bop);

  auto group = [&](int g, auto BUFC) __attribute__((always_inline)) {
    constexpr int BUF = decltype(BUFC)::value;
    const int gn = min(g + 1, G - 1);
    a_read(IntC<BUF>{}, IntC<0>{}, aop[0]);
    a_load(gn, BUF ^ 1);
    // the previous group's last chain, with that group's tile-1 scales and token values
    if (g > 0) fold(dprev, 3, 1, g - 1);
    tok_set(tok);
    s_read(IntC<BUF>{}, IntC<0>{}, sv, bv);
    ds_wait_agpr(aop[0]);
    ds_wait_v4(sv);
    if (ZP) ds_wait_v4(bv);
    __builtin_amdgcn_sched_barrier(0);
    // weight tile 0: chains (0,0) .. (3,0); token tile i + 1 is read during chain (i,0)
    v16i d = chain(bop, aop[0]);
    a_read(IntC<BUF>{}, IntC<1>{}, aop[1]);
    dprev = d;
    __builtin_amdgcn_sched_barrier(0);
    Raw nraw;
    raw_load(nraw, gn);
    Tok ntok;
    tok_load(ntok, gn);
    const uint16_t nsb = s_row[gn];
    const uint32_t nzb = ZP ? static_cast<uint32_t>(z_row[gn >> 1]) : 0u;
    __builtin_amdgcn_sched_barrier(0);
    auto slot0 = [&](auto IC) __attribute__((always_inline)) {
      constexpr int i = decltype(IC)::value;
      ds_wait_agpr(aop[i]);
      const v16i dd = chain(bop, aop[i]);
      fold(dprev, i - 1, 0, g);
      if (i < 3) a_read(IntC<BUF>{}, IntC<(i < 3 ? i + 1 : 3)>{}, aop[i < 3 ? i + 1 : 3]);
      dprev = dd;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, ZP ? 16 : 12, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    };
    slot0(IntC<1>{});
    slot0(IntC<2>{});
    slot0(IntC<3>{});
    // weight tile 1: its B operands replace tile 0's, its scales come after the
    // fold of chain (3,0), which still uses tile 0's
    decode(raw, 1, bop);
    {
      const v16i dd = chain(bop, aop[0]);
      fold(dprev, 3, 0, g);
      dprev = dd;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, ZP ? 16 : 12, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    s_read(IntC<BUF>{}, IntC<1>{}, sv, bv);
    ds_wait_v4(sv);
    if (ZP) ds_wait_v4(bv);
    __builtin_amdgcn_sched_barrier(0);
    auto slot1 = [&](auto IC) __attribute__((always_inline)) {
      constexpr int i = decltype(IC)::value;
      const v16i dd = chain(bop, aop[i]);
      fold(dprev, i - 1, 1, g);
      if (i == 3) decode(nraw, 0, bop);      // next group's tile 0, after the last chain's issue
      dprev = dd;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, i == 3 ? 16 : (ZP ? 16 : 12), 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    };
    slot1(IntC<1>{});
    slot1(IntC<2>{});
    slot1(IntC<3>{});
    raw = nraw;
    tok = ntok;
    __builtin_amdgcn_s_waitcnt(0);     // direct A loads, codes, scales and token values have landed
    stage_scale(nsb, nzb, gn, BUF ^ 1);
    __syncthreads();
  };
  int g = 0;
  for (; g + 1 < G; g += 2) {
    group(g, IntC<0>{});
    group(g + 1, IntC<1>{});
  }
  if (g < G) group(g, IntC<0>{});
  fold(dprev, 3, 1, G - 1);
  if (PARTIALS) return;

  // Epilogue: per token tile, the wave's 32 x 64 block goes through LDS (rows
  // of STAGE_ROW floats), written as lane = token row, read out as 4-value row
  // segments of the output.
  __syncthreads();
  float* stage = reinterpret_cast<float*>(smem + wave * 32 * STAGE_ROW * 4);
  const bool vec = (N & 3) == 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *reinterpret_cast<v4f*>(stage + n * STAGE_ROW + 32 * j + 8 * q + 4 * h) =
            v4f{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int row = 4 * q + (lane >> 4), c4 = 4 * (lane & 15);
      const v4f v4 = *reinterpret_cast<const v4f*>(stage + row * STAGE_ROW + c4);
      const int mm = m0 + 32 * i + row, nn = n0 + 64 * wave + c4;
      if (mm < M) {
        const float v[4] = {v4.x, v4.y, v4.z, v4.w};
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

template <typename TOut, int FX>
hipError_t go_g(const bpw_weights& w, const int8_t* qp, const float* xs, int m, TOut* y, hipStream_t s) {
  const int n = static_cast<int>(w.n), k = static_cast<int>(w.k);
  const int mtiles = (m + BM - 1) / BM, ntiles = (n + BN - 1) / BN;
  gemm_g_kernel<TOut, false, FX><<<mtiles * ntiles, NT, LDS_G_BYTES, s>>>(
      qp, xs, static_cast<const uint8_t*>(w.codes), static_cast<const uint16_t*>(w.scales),
      static_cast<const uint8_t*>(w.zeros), w.scale_dtype == BPW_BF16, m, n, k, y, nullptr, 0, 0, 0, 0, 0, mtiles, 0,
      ntiles);
  return hipGetLastError();
}

template <int FX>
hipError_t go_g_out(const bpw_weights& w, const int8_t* qp, const float* xs, int m, void* y, int y_dtype,
                    hipStream_t s) {
  switch (y_dtype) {
    case BPW_F32: return go_g<float, FX>(w, qp, xs, m, static_cast<float*>(y), s);
    case BPW_F16: return go_g<__half, FX>(w, qp, xs, m, static_cast<__half*>(y), s);
    default: return go_g<uint16_t, FX>(w, qp, xs, m, static_cast<uint16_t*>(y), s);
  }
}

template <int FX>
hipError_t go_g_partials(const bpw_weights& w, const int8_t* qp, int64_t m, int64_t m0, int64_t m1, int64_t n0,
                         int64_t n1, int32_t* out, hipStream_t s) {
  const int n = static_cast<int>(w.n), k = static_cast<int>(w.k);
  const int mt0 = static_cast<int>(m0 / BM), mt1 = static_cast<int>((m1 - 1) / BM);
  const int nt0 = static_cast<int>(n0 / BN), nt1 = static_cast<int>((n1 - 1) / BN);
  const int mtiles = mt1 - mt0 + 1, ntiles = nt1 - nt0 + 1;
  // The partials instance never loads token values.
  gemm_g_kernel<float, true, FX><<<mtiles * ntiles, NT, LDS_G_BYTES, s>>>(
      qp, nullptr, static_cast<const uint8_t*>(w.codes),
      static_cast<const uint16_t*>(w.scales), static_cast<const uint8_t*>(w.zeros), w.scale_dtype == BPW_BF16,
      static_cast<int>(m), n, k, nullptr, out, static_cast<int>(m0), static_cast<int>(m1), static_cast<int>(n0),
      static_cast<int>(n1), mt0, mtiles, nt0, ntiles);
  return hipGetLastError();
}

// The codes-ahead form of the 4-bit weights: K a multiple of 1024 (whole
// 16-byte scale pieces per row, 4-byte zero-point pieces) and the scale and
// zero-point rows of a tile within LDS beside the code slots.
bool deep_ok(int wf, int64_t k) {
  return wf != WF_T2 && k % 1024 == 0 && deep_lds(static_cast<int>(k / 128), wf == WF_I4Z) <= 160 * 1024;
}

template <typename TOut, int WF>
hipError_t go(const bpw_weights& w, const int8_t* qp, const float* xs, int m, TOut* y,
              hipStream_t s) {
  const int n = static_cast<int>(w.n), k = static_cast<int>(w.k);
  const int mtiles = (m + BM - 1) / BM, ntiles = (n + BN - 1) / BN;
  auto launch = [&](auto kern, int lds) {
    allow_lds(kern, lds);
    kern<<<mtiles * ntiles, NT, lds, s>>>(qp, xs, static_cast<const uint8_t*>(w.codes),
                                          static_cast<const uint16_t*>(w.scales), static_cast<const uint8_t*>(w.zeros),
                                          w.scale_dtype == BPW_BF16, m, n, k, y, nullptr, 0, 0, 0, 0, 0, mtiles, 0,
                                          ntiles);
  };
  if constexpr (WF != WF_T2) {
    if (deep_ok(WF, k)) {
      launch(gemm_t2_kernel<TOut, false, WF, true>, deep_lds(k / 128, WF == WF_I4Z));
      return hipGetLastError();
    }
  }
  launch(gemm_t2_kernel<TOut, false, WF>, LDS_BYTES);
  return hipGetLastError();
}

template <int WF>
hipError_t go_out(const bpw_weights& w, const int8_t* qp, const float* xs, int m, void* y, int y_dtype,
                  hipStream_t s) {
  switch (y_dtype) {
    case BPW_F32: return go<float, WF>(w, qp, xs, m, static_cast<float*>(y), s);
    case BPW_F16: return go<__half, WF>(w, qp, xs, m, static_cast<__half*>(y), s);
    default: return go<uint16_t, WF>(w, qp, xs, m, static_cast<uint16_t*>(y), s);
  }
}

template <int WF>
hipError_t go_partials(const bpw_weights& w, const int8_t* qp, int64_t m, int64_t m0, int64_t m1,
                       int64_t n0, int64_t n1, int32_t* out, hipStream_t s) {
  const int n = static_cast<int>(w.n), k = static_cast<int>(w.k);
  const int mt0 = static_cast<int>(m0 / BM), mt1 = static_cast<int>((m1 - 1) / BM);
  const int nt0 = static_cast<int>(n0 / BN), nt1 = static_cast<int>((n1 - 1) / BN);
  const int mtiles = mt1 - mt0 + 1, ntiles = nt1 - nt0 + 1;
  auto launch = [&](auto kern, int lds) {
    allow_lds(kern, lds);
    kern<<<mtiles * ntiles, NT, lds, s>>>(
        qp, nullptr, static_cast<const uint8_t*>(w.codes), static_cast<const uint16_t*>(w.scales),
        static_cast<const uint8_t*>(w.zeros), w.scale_dtype == BPW_BF16, static_cast<int>(m), n, k, nullptr,
        out, static_cast<int>(m0), static_cast<int>(m1), static_cast<int>(n0), static_cast<int>(n1), mt0,
        mtiles, nt0, ntiles);
  };
  // (the partials entry verifies the core the product runs at this K)
  if constexpr (WF != WF_T2) {
    if (deep_ok(WF, k)) {
      launch(gemm_t2_kernel<float, true, WF, true>, deep_lds(k / 128, WF == WF_I4Z));
      return hipGetLastError();
    }
  }
  launch(gemm_t2_kernel<float, true, WF>, LDS_BYTES);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_t2(const bpw_weights& w, const int8_t* q_planes, const float* x_scale,
                          int64_t m, void* y, int y_dtype, hipStream_t s) {
  return go_out<WF_T2>(w, q_planes, x_scale, static_cast<int>(m), y, y_dtype, s);
}

hipError_t launch_gemm_t2_partials(const bpw_weights& w, const int8_t* q_planes, int64_t m,
                                   int64_t m0, int64_t m1, int64_t n0, int64_t n1, int32_t* out,
                                   hipStream_t s) {
  return go_partials<WF_T2>(w, q_planes, m, m0, m1, n0, n1, out, s);
}

hipError_t launch_gemm_w4a8(const bpw_weights& w, const int8_t* q_nibbles, const float* x_scale,
                            int64_t m, void* y, int y_dtype, hipStream_t s) {
  const int mi = static_cast<int>(m);
  return w.fmt == BPW_INT4_ZP ? go_out<WF_I4Z>(w, q_nibbles, x_scale, mi, y, y_dtype, s)
                              : go_out<WF_I4>(w, q_nibbles, x_scale, mi, y, y_dtype, s);
}

hipError_t launch_gemm_g(const bpw_weights& w, const int8_t* q_ordered, const float* x_scale, int64_t m, void* y,
                         int y_dtype, hipStream_t s) {
  const int mi = static_cast<int>(m);
  if (w.fmt == BPW_TERNARY2) return go_g_out<FX_T2G>(w, q_ordered, x_scale, mi, y, y_dtype, s);
  return w.fmt == BPW_INT4_ZP ? go_g_out<FX_AFF_ZP>(w, q_ordered, x_scale, mi, y, y_dtype, s)
                              : go_g_out<FX_AFF_SYM>(w, q_ordered, x_scale, mi, y, y_dtype, s);
}

hipError_t launch_gemm_g_partials(const bpw_weights& w, const int8_t* q_ordered, int64_t m, int64_t m0, int64_t m1,
                                  int64_t n0, int64_t n1, int32_t* out, hipStream_t s) {
  if (w.fmt == BPW_TERNARY2) return go_g_partials<FX_T2G>(w, q_ordered, m, m0, m1, n0, n1, out, s);
  return w.fmt == BPW_INT4_ZP ? go_g_partials<FX_AFF_ZP>(w, q_ordered, m, m0, m1, n0, n1, out, s)
                              : go_g_partials<FX_AFF_SYM>(w, q_ordered, m, m0, m1, n0, n1, out, s);
}

hipError_t launch_gemm_w4a8_partials(const bpw_weights& w, const int8_t* q_nibbles, int64_t m,
                                     int64_t m0, int64_t m1, int64_t n0, int64_t n1, int32_t* out,
                                     hipStream_t s) {
  return w.fmt == BPW_INT4_ZP ? go_partials<WF_I4Z>(w, q_nibbles, m, m0, m1, n0, n1, out, s)
                              : go_partials<WF_I4>(w, q_nibbles, m, m0, m1, n0, n1, out, s);
}

}  // namespace bpw
