// One-time host repack of user weights into the prepared planes (no GPU).
//
// "Kernel experiments: recorded evidence", Test 1: preparation splits the
// 34-byte PQ2 blocks (fp16 scale + 32 code bytes per 128 weights) into one
// aligned code plane and one scale plane, keeping 34 bytes per 128 weights and
// never expanding to dense values; it runs outside any timed call.
// "mate: Marlin-class W4A16 GEMM for mp_31 (SQMMA int4 x fp16) - #6", "Act
// order": the K columns are sorted by group id (stably) and the permutation is
// kept for the activation gather; a g_idx whose sorted groups are not runs of
// exactly one group size is refused with the invariant named.
#include <stdint.h>
#include <string.h>

#include <vector>

#include "../../include/bpw.h"
#include "status.h"

namespace {

constexpr int64_t kGroup = 128;

bool valid_fmt(int fmt) { return fmt == BPW_TERNARY2 || fmt == BPW_INT4_SYM || fmt == BPW_INT4_ZP; }

int check_shape(int fmt, int scale_dtype, int64_t n, int64_t k, int group) {
  if (!valid_fmt(fmt)) return bpw::fail(BPW_EINVAL, "unknown weight format %d", fmt);
  if (scale_dtype != BPW_F16 && scale_dtype != BPW_BF16)
    return bpw::fail(BPW_EINVAL, "scale dtype %d is neither BPW_F16 nor BPW_BF16", scale_dtype);
  if (fmt == BPW_TERNARY2 && scale_dtype != BPW_F16)
    return bpw::fail(BPW_EUNSUPPORTED, "ternary weights carry fp16 scales only");
  if (group != kGroup) return bpw::fail(BPW_EUNSUPPORTED, "group size %d unsupported (only 128)", group);
  if (n < 1 || n > (int64_t(1) << 30)) return bpw::fail(BPW_ESHAPE, "N=%lld outside 1..2^30", (long long)n);
  if (k < kGroup || k % kGroup != 0 || k > (int64_t(1) << 28))
    return bpw::fail(BPW_ESHAPE, "K=%lld must be a positive multiple of 128 (at most 2^28)", (long long)k);
  return BPW_OK;
}

}  // namespace

extern "C" int bpw_packed_sizes(int fmt, int scale_dtype, int64_t n, int64_t k, int group,
                                int has_perm, bpw_sizes* out) {
  if (int st = check_shape(fmt, scale_dtype, n, k, group)) return st;
  if (!out) return bpw::fail(BPW_EINVAL, "out is NULL");
  if (has_perm && fmt == BPW_TERNARY2)
    return bpw::fail(BPW_EUNSUPPORTED, "act-order permutation is supported for 4-bit formats only");
  const int64_t g = k / kGroup;
  out->codes = static_cast<size_t>(fmt == BPW_TERNARY2 ? n * (k / 4) : n * (k / 2));
  out->scales = static_cast<size_t>(n * g * 2);
  out->zeros = fmt == BPW_INT4_ZP ? static_cast<size_t>(n * ((g + 1) / 2)) : 0;
  out->perm = has_perm ? static_cast<size_t>(k * 4) : 0;
  return bpw::ok();
}

extern "C" int bpw_prepare_packed(int fmt, int src_format, int scale_dtype, int64_t n, int64_t k,
                                  int group, const void* src_codes, const void* src_scales,
                                  const uint8_t* src_zeros, const int32_t* g_idx,
                                  void* dst_codes, void* dst_scales, void* dst_zeros,
                                  int32_t* dst_perm) {
  if (int st = check_shape(fmt, scale_dtype, n, k, group)) return st;
  if (src_format != BPW_SRC_PQ2_BLOCKS && src_format != BPW_SRC_PLANES && src_format != BPW_SRC_CODES_U8)
    return bpw::fail(BPW_EINVAL, "unknown source layout %d", src_format);
  if (src_format == BPW_SRC_PQ2_BLOCKS && fmt != BPW_TERNARY2)
    return bpw::fail(BPW_EUNSUPPORTED, "PQ2 blocks hold ternary weights only");
  if (!src_codes) return bpw::fail(BPW_EINVAL, "src_codes is NULL");
  if (src_format == BPW_SRC_PQ2_BLOCKS ? src_scales != nullptr : src_scales == nullptr)
    return bpw::fail(BPW_EINVAL, src_format == BPW_SRC_PQ2_BLOCKS
                                     ? "src_scales must be NULL for PQ2 blocks (scales are inside)"
                                     : "src_scales is NULL");
  const bool zp = fmt == BPW_INT4_ZP;
  if (zp != (src_zeros != nullptr))
    return bpw::fail(BPW_EINVAL, zp ? "INT4_ZP needs src_zeros" : "src_zeros given for a format without zero points");
  if (zp != (dst_zeros != nullptr))
    return bpw::fail(BPW_EINVAL, zp ? "INT4_ZP needs dst_zeros" : "dst_zeros given for a format without zero points");
  if (!dst_codes || !dst_scales) return bpw::fail(BPW_EINVAL, "dst_codes / dst_scales is NULL");
  if ((g_idx != nullptr) != (dst_perm != nullptr))
    return bpw::fail(BPW_EINVAL, "g_idx and dst_perm must be given together");
  if (g_idx && fmt == BPW_TERNARY2)
    return bpw::fail(BPW_EUNSUPPORTED, "act-order permutation is supported for 4-bit formats only");

  const int64_t G = k / kGroup;
  // Act order: validate g_idx and build perm = stable argsort(g_idx) by counting.
  std::vector<int32_t> perm;
  if (g_idx) {
    std::vector<int64_t> count(static_cast<size_t>(G), 0);
    for (int64_t i = 0; i < k; ++i) {
      const int32_t gi = g_idx[i];
      if (gi < 0 || gi >= G)
        return bpw::fail(BPW_EGIDX, "g_idx[%lld] = %d outside 0..%lld", (long long)i, gi, (long long)(G - 1));
      ++count[static_cast<size_t>(gi)];
    }
    for (int64_t g = 0; g < G; ++g)
      if (count[static_cast<size_t>(g)] != kGroup)
        return bpw::fail(BPW_EGIDX, "group %lld has %lld members, expected %lld (sorted groups must be contiguous runs of 128)",
                         (long long)g, (long long)count[static_cast<size_t>(g)], (long long)kGroup);
    perm.resize(static_cast<size_t>(k));
    std::vector<int64_t> next(static_cast<size_t>(G));
    for (int64_t g = 0; g < G; ++g) next[static_cast<size_t>(g)] = g * kGroup;
    for (int64_t i = 0; i < k; ++i) perm[static_cast<size_t>(next[static_cast<size_t>(g_idx[i])]++)] = static_cast<int32_t>(i);
  }

  const uint8_t* sc = static_cast<const uint8_t*>(src_codes);
  uint8_t* dc = static_cast<uint8_t*>(dst_codes);
  uint8_t* ds = static_cast<uint8_t*>(dst_scales);

  // Range checks first, so that a refused call writes nothing.
  if (src_format == BPW_SRC_CODES_U8) {
    const uint32_t limit = fmt == BPW_TERNARY2 ? 3 : 15;
    for (int64_t i = 0; i < n * k; ++i)
      if (sc[i] > limit)
        return bpw::fail(BPW_EINVAL, "code %u at row %lld col %lld exceeds %u", sc[i],
                         (long long)(i / k), (long long)(i % k), limit);
    if (zp)
      for (int64_t i = 0; i < n * G; ++i)
        if (src_zeros[i] > 15)
          return bpw::fail(BPW_EINVAL, "zero point %u at row %lld group %lld exceeds 15",
                           src_zeros[i], (long long)(i / G), (long long)(i % G));
  }

  if (fmt == BPW_TERNARY2) {
    const int64_t rb = k / 4;                 // code bytes per row
    for (int64_t r = 0; r < n; ++r) {
      uint8_t* out = dc + r * rb;
      if (src_format == BPW_SRC_PQ2_BLOCKS) {
        const uint8_t* blk = sc + r * G * 34;
        for (int64_t g = 0; g < G; ++g) {
          memcpy(ds + (r * G + g) * 2, blk + g * 34, 2);          // fp16 scale, little-endian
          memcpy(out + g * 32, blk + g * 34 + 2, 32);
        }
      } else if (src_format == BPW_SRC_PLANES) {
        memcpy(out, sc + r * rb, static_cast<size_t>(rb));
      } else {
        const uint8_t* in = sc + r * k;
        for (int64_t b = 0; b < rb; ++b) {
          uint32_t v = 0;
          for (int t = 0; t < 4; ++t) {
            v |= static_cast<uint32_t>(in[4 * b + t]) << (2 * t);
          }
          out[b] = static_cast<uint8_t>(v);
        }
      }
    }
    if (src_format != BPW_SRC_PQ2_BLOCKS) memcpy(ds, src_scales, static_cast<size_t>(n * G * 2));
    return bpw::ok();
  }

  // 4-bit formats.
  const int64_t rb = k / 2;
  for (int64_t r = 0; r < n; ++r) {
    uint8_t* out = dc + r * rb;
    if (src_format == BPW_SRC_PLANES && perm.empty()) {
      memcpy(out, sc + r * rb, static_cast<size_t>(rb));
      continue;
    }
    for (int64_t b = 0; b < rb; ++b) {
      uint32_t v = 0;
      for (int t = 0; t < 2; ++t) {
        const int64_t j = 2 * b + t;
        const int64_t col = perm.empty() ? j : perm[static_cast<size_t>(j)];
        uint32_t c;
        if (src_format == BPW_SRC_PLANES) {
          c = (sc[r * rb + col / 2] >> (4 * (col & 1))) & 15u;
        } else {
          c = sc[r * k + col];
        }
        v |= c << (4 * t);
      }
      out[b] = static_cast<uint8_t>(v);
    }
  }
  memcpy(ds, src_scales, static_cast<size_t>(n * G * 2));
  if (zp) {
    const int64_t zb = (G + 1) / 2;
    uint8_t* dz = static_cast<uint8_t*>(dst_zeros);
    for (int64_t r = 0; r < n; ++r) {
      for (int64_t b = 0; b < zb; ++b) {
        uint32_t v = 0;
        for (int t = 0; t < 2; ++t) {
          const int64_t g = 2 * b + t;
          if (g >= G) break;
          uint32_t z;
          if (src_format == BPW_SRC_PLANES) {
            z = (src_zeros[r * zb + b] >> (4 * t)) & 15u;
          } else {
            z = src_zeros[r * G + g];
          }
          v |= z << (4 * t);
        }
        dz[r * zb + b] = static_cast<uint8_t>(v);
      }
    }
  }
  if (!perm.empty()) memcpy(dst_perm, perm.data(), static_cast<size_t>(k) * 4);
  return bpw::ok();
}
