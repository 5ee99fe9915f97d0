// bpw_gemv_packed_scratch: the decode product for callers that cannot allocate
// device memory (code under HIP graph capture, tight serving loops, harnesses
// that forbid hipMalloc). It is bpw_gemv_packed with its workspace taken from
// a fixed device array of this library instead of a caller buffer.
//
// The array lives in device memory for as long as the library is loaded; each
// GPU the library runs on holds its own copy at its own address. In host code
// the array's name is only a host-side stand-in, so the device address of the
// copy on each GPU is resolved once per device, with that device current, by
// hipGetSymbolAddress, and only that address is ever given to kernels.
//
// Nothing here allocates: no hipMalloc, no hipFree, no allocating library call.
// The kernels fully write every workspace byte they later read (split-K slices,
// the act-order gather), so no part of the array has to start at zero and the
// previous call's contents are never read. Calls that overlap on one GPU (two
// streams, two threads) share the array and race.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "../../include/bpw.h"
#include "product.h"
#include "status.h"

static __device__ __align__(256) unsigned char scratch[BPW_SCRATCH_BYTES];

namespace bpw {
namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mu;
std::atomic<void*> g_scratch[kMaxDevices];

// Device address of this GPU's copy of the array, resolved on first use.
int scratch_ptr(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(BPW_EHIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(BPW_EUNSUPPORTED, "device index %d out of range", dev);
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_mu);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (!p) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess || !p)
        return fail(BPW_EHIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return BPW_OK;
}

}  // namespace
}  // namespace bpw

using namespace bpw;

extern "C" int bpw_gemv_packed_scratch(const bpw_weights* w, const void* x, int x_dtype,
                                       const float* x_scale, int64_t m, void* y, int y_dtype,
                                       void* stream) {
  if (int st = check_product_args(w, x, x_dtype, x_scale, m, y, y_dtype)) return st;
  const size_t need = workspace_need(w, m, x_dtype, BPW_PATH_GEMV);
  if (need > BPW_SCRATCH_BYTES)
    return fail(BPW_ESHAPE,
                "this call needs %zu bytes of workspace; the fixed scratch holds %d (use bpw_gemv_packed "
                "with a caller workspace)",
                need, BPW_SCRATCH_BYTES);
  if (int st = check_current_device(stream)) return st;
  void* ws = nullptr;
  if (need > 0) {
    if (int st = scratch_ptr(&ws)) return st;
  }
  return run_product(true, w, x, x_dtype, x_scale, m, y, y_dtype, ws, need > 0 ? BPW_SCRATCH_BYTES : 0, stream);
}
