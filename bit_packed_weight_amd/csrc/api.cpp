// C ABI: argument validation, workspace sizing and kernel dispatch.
// Every check runs on the host before any HIP call, so a refused call launches
// nothing and leaves outputs untouched.
#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <string>

#include "../../include/bpw.h"
#include "launch.h"
#include "product.h"
#include "status.h"

namespace bpw {

namespace {
thread_local std::string g_error;
constexpr size_t kWsAlign = 256;

size_t round_up(size_t v) { return (v + kWsAlign - 1) / kWsAlign * kWsAlign; }
bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }
bool is_int4(int fmt) { return fmt == BPW_INT4_SYM || fmt == BPW_INT4_ZP; }
bool is_out_dtype(int d) { return d == BPW_F32 || d == BPW_F16 || d == BPW_BF16; }

// The device a call runs on: the current device, which must also be the
// stream's device (kernels launch on the stream, and the workspace and operand
// pointers are the caller's allocations on it); gfx950 checked once per device
// (the kernels are compiled for gfx950 only).
int check_device(hipStream_t stream) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(BPW_EHIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (stream) {
    hipDevice_t sdev = 0;
    e = hipStreamGetDevice(stream, &sdev);
    if (e != hipSuccess) return fail(BPW_EHIP, "hipStreamGetDevice: %s", hipGetErrorString(e));
    if (static_cast<int>(sdev) != dev)
      return fail(BPW_EINVAL, "the stream belongs to device %d but device %d is current", static_cast<int>(sdev), dev);
  }
  static std::mutex mu;
  static int checked[64] = {0};   // 0 unknown, 1 ok, 2 wrong architecture
  std::lock_guard<std::mutex> lock(mu);
  if (dev < 0 || dev >= 64) return fail(BPW_EUNSUPPORTED, "device index %d out of range", dev);
  if (checked[dev] == 0) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return fail(BPW_EHIP, "hipGetDeviceProperties: %s", hipGetErrorString(e));
    checked[dev] = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    if (checked[dev] == 2)
      return fail(BPW_EUNSUPPORTED, "device %d is %s; this library is built for gfx950 only", dev, prop.gcnArchName);
  }
  if (checked[dev] == 2) return fail(BPW_EUNSUPPORTED, "device %d is not gfx950", dev);
  return BPW_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(BPW_EHIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

}  // namespace

int check_weights(const bpw_weights* w) {
  if (!w) return fail(BPW_EINVAL, "weights descriptor is NULL");
  if (w->fmt != BPW_TERNARY2 && !is_int4(w->fmt)) return fail(BPW_EINVAL, "unknown weight format %d", w->fmt);
  if (w->group != 128) return fail(BPW_EUNSUPPORTED, "group size %d unsupported (only 128)", w->group);
  if (w->reserved != 0) return fail(BPW_EINVAL, "reserved field must be 0");
  if (w->n < 1 || w->n > (int64_t(1) << 30)) return fail(BPW_ESHAPE, "N=%lld outside 1..2^30", (long long)w->n);
  if (w->k < 128 || w->k % 128 != 0 || w->k > (int64_t(1) << 28))
    return fail(BPW_ESHAPE, "K=%lld must be a positive multiple of 128 (at most 2^28)", (long long)w->k);
  if (w->scale_dtype != BPW_F16 && w->scale_dtype != BPW_BF16)
    return fail(BPW_EINVAL, "scale dtype %d is neither BPW_F16 nor BPW_BF16", w->scale_dtype);
  if (w->fmt == BPW_TERNARY2 && w->scale_dtype != BPW_F16)
    return fail(BPW_EUNSUPPORTED, "ternary weights carry fp16 scales only");
  if (!w->codes || !w->scales) return fail(BPW_EINVAL, "codes / scales plane is NULL");
  if (!aligned(w->codes, 16)) return fail(BPW_EALIGN, "codes plane must be 16-byte aligned");
  if (!aligned(w->scales, 16)) return fail(BPW_EALIGN, "scales plane must be 16-byte aligned");
  if (w->zeros && !aligned(w->zeros, 16)) return fail(BPW_EALIGN, "zero-point plane must be 16-byte aligned");
  if ((w->fmt == BPW_INT4_ZP) != (w->zeros != nullptr))
    return fail(BPW_EINVAL, w->fmt == BPW_INT4_ZP ? "INT4_ZP needs a zero-point plane" : "zero-point plane given for a format without zero points");
  if (w->perm && w->fmt == BPW_TERNARY2)
    return fail(BPW_EUNSUPPORTED, "act-order permutation is supported for 4-bit formats only");
  if (w->perm && !aligned(w->perm, 4)) return fail(BPW_EALIGN, "perm must be 4-byte aligned");
  return BPW_OK;
}

namespace {

int check_product(const bpw_weights* w, const void* x, int x_dtype, const float* x_scale,
                  int64_t m, void* y, int y_dtype) {
  if (int st = check_weights(w)) return st;
  if (m < 1 || m > (int64_t(1) << 30)) return fail(BPW_ESHAPE, "M=%lld outside 1..2^30", (long long)m);
  if (!x || !y) return fail(BPW_EINVAL, "x / y is NULL");
  if (!is_out_dtype(y_dtype)) return fail(BPW_EUNSUPPORTED, "output dtype %d unsupported (F32, F16, BF16)", y_dtype);
  if (w->fmt == BPW_TERNARY2 && (x_dtype == BPW_F32 || x_dtype == BPW_F16 || x_dtype == BPW_BF16)) {
    // the complete one-token call: the row quantiser fused into the decode GEMV
    if (x_scale) return fail(BPW_EINVAL, "x_scale must be NULL: the call quantises the activations itself");
    if (!gemv_t2_fused_fits(m, w->k))
      return fail(BPW_EUNSUPPORTED,
                  "ternary weights quantise fp32/fp16/bf16 activations inside the call only at M = 1, K <= 16384 "
                  "(M=%lld, K=%lld given); quantise with bpw_quantize_rows first",
                  (long long)m, (long long)w->k);
  } else if (w->fmt == BPW_TERNARY2) {
    if (x_dtype != BPW_I8 && x_dtype != BPW_I8G)
      return fail(BPW_EUNSUPPORTED, "ternary weights take int8 activations (x_dtype %d given)", x_dtype);
    if (!x_scale) return fail(BPW_EINVAL, x_dtype == BPW_I8 ? "int8 activations need x_scale [M]"
                                                            : "int8 activations need x_scale [M][K/128]");
    if (!aligned(x_scale, 4)) return fail(BPW_EALIGN, "x_scale must be 4-byte aligned");
  } else if (x_dtype == BPW_I8) {
    // "TensorFold PR #1176": 4-bit weights against int8 activations on the int8 matrix core.
    if (!x_scale) return fail(BPW_EINVAL, "int8 activations need x_scale [M]");
    if (!aligned(x_scale, 4)) return fail(BPW_EALIGN, "x_scale must be 4-byte aligned");
  } else if (x_dtype == BPW_I8GS) {
    // The same page's affine form: (a, sum) per row and weight group.
    if (!x_scale) return fail(BPW_EINVAL, "BPW_I8GS activations need x_scale [M][K/128][2]");
    if (!aligned(x_scale, 8)) return fail(BPW_EALIGN, "x_scale of BPW_I8GS must be 8-byte aligned");
  } else {
    if (x_dtype != BPW_F16 && x_dtype != BPW_BF16)
      return fail(BPW_EUNSUPPORTED, "4-bit weights take fp16, bf16 or int8 (row scale) activations (x_dtype %d given)",
                  x_dtype);
    if (x_dtype != w->scale_dtype)
      return fail(BPW_EUNSUPPORTED, "4-bit weights need scale dtype == activation dtype");
    if (x_scale) return fail(BPW_EINVAL, "x_scale must be NULL for fp16/bf16 activations");
  }
  if (!aligned(x, 16)) return fail(BPW_EALIGN, "x must be 16-byte aligned");
  if (!aligned(y, y_dtype == BPW_F32 ? 4 : 2)) return fail(BPW_EALIGN, "y is misaligned for its dtype");
  return BPW_OK;
}

}  // namespace

int check_product_args(const bpw_weights* w, const void* x, int x_dtype, const float* x_scale, int64_t m,
                       void* y, int y_dtype) {
  return check_product(w, x, x_dtype, x_scale, m, y, y_dtype);
}

int check_current_device(void* stream) { return check_device(static_cast<hipStream_t>(stream)); }

// Workspace bytes for (weights, M, activation type, entry).
size_t workspace_need(const bpw_weights* w, int64_t m, int x_dtype, int entry) {
  const size_t mk = static_cast<size_t>(m) * static_cast<size_t>(w->k);
  if (w->fmt == BPW_TERNARY2 && (x_dtype == BPW_F32 || x_dtype == BPW_F16 || x_dtype == BPW_BF16))
    return 0;                                  // quantised inside the decode kernel
  if (w->fmt == BPW_TERNARY2) {
    if (x_dtype == BPW_I8G && entry == BPW_PATH_GEMV && gemv_t2_group_fits(m, w->k))
      return 0;                                // decode kernels, no staging
    if (x_dtype != BPW_I8G && entry == BPW_PATH_GEMV && gemv_t2_fits(m, w->k))   // fp32 split-K slices for long K
      return round_up(gemv_t2_split_bytes(m, w->n, w->k, false));
    return round_up(mk);                       // plane-ordered int8 activations
  }
  if (x_dtype == BPW_I8 || x_dtype == BPW_I8GS) return round_up(mk);  // nibble-ordered int8 activations
  // gathered 16-bit activations, then the fp32 split-K slices of a long-K decode
  const size_t gather = w->perm ? round_up(mk * 2) : 0;
  if (entry == BPW_PATH_GEMV && gemv_w4_fits(m, w->k)) return gather + round_up(gemv_w4_split_bytes(m, w->n, w->k));
  return gather;
}

namespace {

int check_workspace(const bpw_weights* w, int64_t m, int x_dtype, int entry, void* ws, size_t ws_bytes) {
  const size_t need = workspace_need(w, m, x_dtype, entry);
  if (need == 0) return BPW_OK;
  if (!ws) return fail(BPW_EINVAL, "this call needs a %zu-byte device workspace", need);
  if (!aligned(ws, kWsAlign)) return fail(BPW_EALIGN, "workspace must be 256-byte aligned");
  if (ws_bytes < need) return fail(BPW_ESHAPE, "workspace has %zu bytes, needs %zu", ws_bytes, need);
  return BPW_OK;
}

}  // namespace

int run_product(bool gemv, const bpw_weights* w, const void* x, int x_dtype, const float* x_scale,
                int64_t m, void* y, int y_dtype, void* ws, size_t ws_bytes, void* stream) {
  const int entry = gemv ? BPW_PATH_GEMV : BPW_PATH_GEMM;
  if (int st = check_product(w, x, x_dtype, x_scale, m, y, y_dtype)) return st;
  if (is_int4(w->fmt) && (x_dtype == BPW_I8 || x_dtype == BPW_I8GS) && gemv)
    return fail(BPW_EUNSUPPORTED, "4-bit weights with int8 activations run through bpw_gemm_packed only");
  const bool t2_float = w->fmt == BPW_TERNARY2 && (x_dtype == BPW_F32 || x_dtype == BPW_F16 || x_dtype == BPW_BF16);
  if (t2_float && !gemv)
    return fail(BPW_EUNSUPPORTED, "ternary weights with fp32/fp16/bf16 activations run through bpw_gemv_packed only");
  if (int st = check_workspace(w, m, x_dtype, entry, ws, ws_bytes)) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (int st = check_device(s)) return st;
  if (is_int4(w->fmt) && (x_dtype == BPW_I8 || x_dtype == BPW_I8GS)) {
    int8_t* qn = static_cast<int8_t*>(ws);
    if (int st = hip_status(launch_int8_nibbles(static_cast<const int8_t*>(x), w->perm, m, w->k, qn, s),
                            "int8 nibble reorder launch"))
      return st;
    if (x_dtype == BPW_I8GS)   // "TensorFold PR #1176": s * a * (code . q) + b * sum(x) per group
      return hip_status(launch_gemm_g(*w, qn, x_scale, m, y, y_dtype, s), "4-bit x int8 affine GEMM launch");
    return hip_status(launch_gemm_w4a8(*w, qn, x_scale, m, y, y_dtype, s), "4-bit x int8 GEMM launch");
  }
  if (t2_float)
    return hip_status(launch_gemv_t2_fused(*w, x, x_dtype, y, y_dtype, s), "ternary quantise-and-GEMV launch");
  if (w->fmt == BPW_TERNARY2) {
    const int8_t* q = static_cast<const int8_t*>(x);
    if (x_dtype == BPW_I8G && gemv && gemv_t2_group_fits(m, w->k))
      return hip_status(launch_gemv_t2(*w, q, x_scale, m, y, y_dtype, true, nullptr, 0, s), "ternary GEMV launch");
    if (x_dtype == BPW_I8G) {
      // "Kernel experiments", Test 7: partial * x_scale * w_scale per 128-group, on the
      // prefill kernel with one activation scale per (row, group).
      int8_t* qp = static_cast<int8_t*>(ws);
      if (int st = hip_status(launch_int8_planes(q, m, w->k, qp, s), "int8 plane reorder launch")) return st;
      return hip_status(launch_gemm_g(*w, qp, x_scale, m, y, y_dtype, s), "ternary GEMM launch");
    }
    if (gemv && gemv_t2_fits(m, w->k))
      return hip_status(launch_gemv_t2(*w, q, x_scale, m, y, y_dtype, false, ws, ws_bytes, s), "ternary GEMV launch");
    int8_t* qp = static_cast<int8_t*>(ws);
    if (int st = hip_status(launch_int8_planes(q, m, w->k, qp, s), "int8 plane reorder launch")) return st;
    return hip_status(launch_gemm_t2(*w, qp, x_scale, m, y, y_dtype, s), "ternary GEMM launch");
  }
  if (gemv && gemv_w4_perm_fits(*w, m, x))
    return hip_status(launch_gemv_w4_perm(*w, x, x_dtype, m, y, y_dtype, s), "4-bit act-order GEMV launch");
  const void* xs = x;
  size_t used = 0;
  if (w->perm) {
    uint16_t* xp = static_cast<uint16_t*>(ws);
    if (int st = hip_status(launch_gather_cols(static_cast<const uint16_t*>(x), w->perm, m, w->k, xp, s), "act-order gather launch"))
      return st;
    xs = xp;
    used = round_up(static_cast<size_t>(m) * w->k * 2);
  }
  if (gemv && gemv_w4_fits(m, w->k)) {
    float* part = gemv_w4_split_bytes(m, w->n, w->k) > 0 ? reinterpret_cast<float*>(static_cast<char*>(ws) + used) : nullptr;
    return hip_status(launch_gemv_w4(*w, xs, x_dtype, m, y, y_dtype, part, s), "4-bit GEMV launch");
  }
  return hip_status(launch_gemm_w4(*w, xs, x_dtype, m, y, y_dtype, s), "4-bit GEMM launch");
}

int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_error = buf;
  return status;
}

int ok() {
  g_error.clear();
  return BPW_OK;
}

}  // namespace bpw

using namespace bpw;

extern "C" int bpw_version(void) { return 100; }

extern "C" const char* bpw_last_error(void) { return g_error.c_str(); }

extern "C" int bpw_quantize_rows(const void* x, int x_dtype, int64_t m, int64_t k, int8_t* q,
                                 float* x_scale, void* stream) {
  if (!x || !q || !x_scale) return fail(BPW_EINVAL, "x / q / x_scale is NULL");
  if (x_dtype != BPW_F32 && x_dtype != BPW_F16 && x_dtype != BPW_BF16)
    return fail(BPW_EUNSUPPORTED, "quantiser input dtype %d unsupported (F32, F16, BF16)", x_dtype);
  if (m < 1 || m > (int64_t(1) << 30) || k < 1 || k > (int64_t(1) << 30))
    return fail(BPW_ESHAPE, "M=%lld, K=%lld must be in 1..2^30", (long long)m, (long long)k);
  if (!aligned(x, x_dtype == BPW_F32 ? 4 : 2) || !aligned(x_scale, 4))
    return fail(BPW_EALIGN, "x / x_scale misaligned for their dtypes");
  if (int st = check_device(static_cast<hipStream_t>(stream))) return st;
  return hip_status(launch_quantize_rows(x, x_dtype, m, k, q, x_scale, static_cast<hipStream_t>(stream)),
                    "quantiser launch");
}

extern "C" int bpw_quantize_groups(const void* x, int x_dtype, int64_t m, int64_t k, int8_t* q,
                                   float* x_scale, void* stream) {
  if (!x || !q || !x_scale) return fail(BPW_EINVAL, "x / q / x_scale is NULL");
  if (x_dtype != BPW_F32 && x_dtype != BPW_F16 && x_dtype != BPW_BF16)
    return fail(BPW_EUNSUPPORTED, "quantiser input dtype %d unsupported (F32, F16, BF16)", x_dtype);
  if (m < 1 || m > (int64_t(1) << 30) || k < 128 || k > (int64_t(1) << 30) || k % 128 != 0)
    return fail(BPW_ESHAPE, "M=%lld must be in 1..2^30 and K=%lld a multiple of 128 up to 2^30", (long long)m,
                (long long)k);
  if (!aligned(x, x_dtype == BPW_F32 ? 4 : 2) || !aligned(q, 16) || !aligned(x_scale, 4))
    return fail(BPW_EALIGN, "x / q / x_scale misaligned (q must be 16-byte aligned)");
  if (int st = check_device(static_cast<hipStream_t>(stream))) return st;
  return hip_status(launch_quantize_groups(x, x_dtype, m, k, q, x_scale, static_cast<hipStream_t>(stream)),
                    "group quantiser launch");
}

extern "C" int bpw_quantize_groups_sums(const void* x, int x_dtype, int64_t m, int64_t k, const int32_t* perm,
                                        int8_t* q, float* x_scale_sum, void* stream) {
  if (!x || !q || !x_scale_sum) return fail(BPW_EINVAL, "x / q / x_scale_sum is NULL");
  if (x_dtype != BPW_F32 && x_dtype != BPW_F16 && x_dtype != BPW_BF16)
    return fail(BPW_EUNSUPPORTED, "quantiser input dtype %d unsupported (F32, F16, BF16)", x_dtype);
  if (m < 1 || m > (int64_t(1) << 30) || k < 128 || k > (int64_t(1) << 30) || k % 128 != 0)
    return fail(BPW_ESHAPE, "M=%lld must be in 1..2^30 and K=%lld a multiple of 128 up to 2^30", (long long)m,
                (long long)k);
  if (!aligned(x, x_dtype == BPW_F32 ? 4 : 2) || !aligned(q, 16) || !aligned(x_scale_sum, 8) ||
      (perm && !aligned(perm, 4)))
    return fail(BPW_EALIGN, "x / q / x_scale_sum / perm misaligned (q 16-byte, x_scale_sum 8-byte)");
  if (int st = check_device(static_cast<hipStream_t>(stream))) return st;
  return hip_status(launch_quantize_groups_sums(x, x_dtype, perm, m, k, q, x_scale_sum,
                                                static_cast<hipStream_t>(stream)),
                    "group quantiser (with sums) launch");
}

extern "C" int bpw_workspace_size(const bpw_weights* w, int64_t m, int x_dtype, int entry,
                                  size_t* bytes) {
  if (int st = check_weights(w)) return st;
  if (!bytes) return fail(BPW_EINVAL, "bytes is NULL");
  if (entry != BPW_PATH_GEMV && entry != BPW_PATH_GEMM) return fail(BPW_EINVAL, "unknown entry %d", entry);
  if (m < 1 || m > (int64_t(1) << 30)) return fail(BPW_ESHAPE, "M=%lld outside 1..2^30", (long long)m);
  *bytes = workspace_need(w, m, x_dtype, entry);
  return ok();
}

extern "C" int bpw_gemv_packed(const bpw_weights* w, const void* x, int x_dtype,
                               const float* x_scale, int64_t m, void* y, int y_dtype,
                               void* workspace, size_t workspace_bytes, void* stream) {
  return run_product(true, w, x, x_dtype, x_scale, m, y, y_dtype, workspace, workspace_bytes, stream);
}

extern "C" int bpw_gemm_packed(const bpw_weights* w, const void* x, int x_dtype,
                               const float* x_scale, int64_t m, void* y, int y_dtype,
                               void* workspace, size_t workspace_bytes, void* stream) {
  return run_product(false, w, x, x_dtype, x_scale, m, y, y_dtype, workspace, workspace_bytes, stream);
}

extern "C" int bpw_partials(const bpw_weights* w, const int8_t* q, int64_t m, int path,
                            int64_t m0, int64_t m1, int64_t n0, int64_t n1, int32_t* out,
                            void* workspace, size_t workspace_bytes, void* stream) {
  if (int st = check_weights(w)) return st;
  if (!q || !out) return fail(BPW_EINVAL, "q / out is NULL");
  if (!aligned(q, 16)) return fail(BPW_EALIGN, "q must be 16-byte aligned");
  if (!aligned(out, 4)) return fail(BPW_EALIGN, "out must be 4-byte aligned");
  if (m < 1 || m > (int64_t(1) << 30)) return fail(BPW_ESHAPE, "M=%lld outside 1..2^30", (long long)m);
  if (!(0 <= m0 && m0 < m1 && m1 <= m) || !(0 <= n0 && n0 < n1 && n1 <= w->n))
    return fail(BPW_ESHAPE, "window [%lld,%lld) x [%lld,%lld) outside M=%lld, N=%lld", (long long)m0,
                (long long)m1, (long long)n0, (long long)n1, (long long)m, (long long)w->n);
  if (path != BPW_PATH_GEMV && path != BPW_PATH_GEMM && path != BPW_PATH_GEMM_RAW)
    return fail(BPW_EINVAL, "unknown path %d", path);
  if (w->fmt != BPW_TERNARY2 && path == BPW_PATH_GEMV)
    return fail(BPW_EUNSUPPORTED, "partials of 4-bit weights come from the GEMM cores only");
  if (path == BPW_PATH_GEMV && !gemv_t2_fits(m, w->k))
    return fail(BPW_ESHAPE, "the GEMV core takes M <= 32");
  if (path != BPW_PATH_GEMV) {
    if (int st = check_workspace(w, m, BPW_I8, BPW_PATH_GEMM, workspace, workspace_bytes)) return st;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (int st = check_device(s)) return st;
  if (path == BPW_PATH_GEMV)
    return hip_status(launch_gemv_t2_partials(*w, q, m, m0, m1, n0, n1, out, s), "GEMV partials launch");
  int8_t* qp = static_cast<int8_t*>(workspace);
  if (w->fmt != BPW_TERNARY2) {
    if (int st = hip_status(launch_int8_nibbles(q, w->perm, m, w->k, qp, s), "int8 nibble reorder launch")) return st;
    if (path == BPW_PATH_GEMM_RAW)
      return hip_status(launch_gemm_g_partials(*w, qp, m, m0, m1, n0, n1, out, s), "GEMM partials launch");
    return hip_status(launch_gemm_w4a8_partials(*w, qp, m, m0, m1, n0, n1, out, s), "GEMM partials launch");
  }
  if (int st = hip_status(launch_int8_planes(q, m, w->k, qp, s), "int8 plane reorder launch")) return st;
  if (path == BPW_PATH_GEMM_RAW)
    return hip_status(launch_gemm_g_partials(*w, qp, m, m0, m1, n0, n1, out, s), "GEMM partials launch");
  return hip_status(launch_gemm_t2_partials(*w, qp, m, m0, m1, n0, n1, out, s), "GEMM partials launch");
}

extern "C" int64_t bpw_probe_blocks(size_t bytes) { return probe_blocks(bytes); }

extern "C" int bpw_probe(int kind, const void* src, void* dst, size_t bytes, void* stream) {
  if (kind != BPW_PROBE_READ && kind != BPW_PROBE_COPY) return fail(BPW_EINVAL, "unknown probe %d", kind);
  if (!src || !dst) return fail(BPW_EINVAL, "src / dst is NULL");
  if (bytes == 0 || bytes % 16) return fail(BPW_ESHAPE, "bytes must be a positive multiple of 16");
  if (!aligned(src, 16) || !aligned(dst, kind == BPW_PROBE_COPY ? 16 : 4))
    return fail(BPW_EALIGN, "src / dst misaligned");
  if (int st = check_device(static_cast<hipStream_t>(stream))) return st;
  return hip_status(launch_probe(kind, src, dst, bytes, static_cast<hipStream_t>(stream)), "probe launch");
}
