// Direct global -> LDS copies (prefill GEMMs, act-order decode staging).
#pragma once

#include <stdint.h>

namespace bpw {

// 16 bytes per lane from global memory straight into LDS (gfx950
// global_load_lds_dwordx4): lane i's 16 bytes land at LDS byte address
// lds_base + 16 * i (lds_base must be wave-uniform; it goes through m0).
// Issued from inline assembly so that the compiler does not add its own
// conservative waits on later LDS reads; the caller waits (vmcnt) and
// synchronises before the data is read. The block keeps m0 as it found it
// (saved and restored in a scratch SGPR), and puts one wait state between the
// m0 write and the load, which reads m0 as it issues (a gfx9 hazard the
// compiler cannot see inside inline assembly).
__device__ __forceinline__ void lds_dma16(const void* src, uint32_t lds_base) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %2, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds_base), "v"(src)
      : "memory");
}

// The same with 4 bytes per lane (global_load_lds_dword): lane i's 4 bytes
// land at lds_base + 4 * i.
__device__ __forceinline__ void lds_dma4(const void* src, uint32_t lds_base) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dword %2, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds_base), "v"(src)
      : "memory");
}

// Wait until at most N vector memory operations of this wave are outstanding
// (gfx9 s_waitcnt: vmcnt in bits 3:0 and 15:14; expcnt 7 and lgkmcnt 15 mean
// no wait on those counters). Operations complete in issue order, so this
// waits for everything issued before the last N.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt holds 0..63");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

}  // namespace bpw
