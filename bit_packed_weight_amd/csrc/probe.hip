// HBM probes: a plain streaming read and a plain copy of a known byte count.
// They calibrate the hardware byte counters (bytes fetched / written per
// dispatch) and give the achievable streaming rate on this device, in the
// spirit of "Kernel experiments: recorded evidence", Test 24 (copy-only load
// probes of the code bytes, no arithmetic).
#include "device.h"
#include "launch.h"

namespace bpw {
namespace {

constexpr int kThreads = 256;
constexpr int kPerThread = 8;   // 16-byte loads per thread
constexpr size_t kBlockBytes = static_cast<size_t>(kThreads) * kPerThread * 16;

__global__ __launch_bounds__(kThreads) void probe_read_kernel(const v4u* __restrict__ src,
                                                              size_t n16,
                                                              uint32_t* __restrict__ dst) {
  const size_t base = static_cast<size_t>(blockIdx.x) * kThreads * kPerThread;
  v4u v[kPerThread];
#pragma unroll
  for (int i = 0; i < kPerThread; ++i) {
    const size_t idx = base + static_cast<size_t>(i) * kThreads + threadIdx.x;
    v[i] = idx < n16 ? __builtin_nontemporal_load(src + idx) : v4u{0, 0, 0, 0};   // streaming, as the GEMVs
  }
  uint32_t x = 0;
#pragma unroll
  for (int i = 0; i < kPerThread; ++i) x ^= v[i].x ^ v[i].y ^ v[i].z ^ v[i].w;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x ^= __shfl_xor(x, off);
  __shared__ uint32_t red[kThreads / 64];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  if (threadIdx.x == 0) dst[blockIdx.x] = red[0] ^ red[1] ^ red[2] ^ red[3];
}

__global__ __launch_bounds__(kThreads) void probe_copy_kernel(const v4u* __restrict__ src,
                                                              size_t n16,
                                                              v4u* __restrict__ dst) {
  const size_t base = static_cast<size_t>(blockIdx.x) * kThreads * kPerThread;
  v4u v[kPerThread];
#pragma unroll
  for (int i = 0; i < kPerThread; ++i) {
    const size_t idx = base + static_cast<size_t>(i) * kThreads + threadIdx.x;
    if (idx < n16) v[i] = src[idx];
  }
#pragma unroll
  for (int i = 0; i < kPerThread; ++i) {
    const size_t idx = base + static_cast<size_t>(i) * kThreads + threadIdx.x;
    if (idx < n16) dst[idx] = v[i];
  }
}

}  // namespace

int64_t probe_blocks(size_t bytes) {
  return static_cast<int64_t>((bytes + kBlockBytes - 1) / kBlockBytes);
}

hipError_t launch_probe(int kind, const void* src, void* dst, size_t bytes, hipStream_t s) {
  const size_t n16 = bytes / 16;
  const int64_t blocks = probe_blocks(bytes);
  if (kind == BPW_PROBE_READ)
    probe_read_kernel<<<static_cast<unsigned>(blocks), kThreads, 0, s>>>(
        static_cast<const v4u*>(src), n16, static_cast<uint32_t*>(dst));
  else
    probe_copy_kernel<<<static_cast<unsigned>(blocks), kThreads, 0, s>>>(
        static_cast<const v4u*>(src), n16, static_cast<v4u*>(dst));
  return hipGetLastError();
}

}  // namespace bpw
