// Host-side launchers implemented next to their kernels. Arguments are already
// validated by the C-ABI layer (api.cpp); launchers only pick a configuration
// and launch on the given stream.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/bpw.h"

namespace bpw {

// Activation operand preparation (quant.hip).
hipError_t launch_quantize_rows(const void* x, int x_dtype, int64_t m, int64_t k, int8_t* q,
                                float* x_scale, hipStream_t s);
// One scale per (row, 128-group): x_scale [M][K/128]. K % 128 == 0.
hipError_t launch_quantize_groups(const void* x, int x_dtype, int64_t m, int64_t k, int8_t* q,
                                  float* x_scale, hipStream_t s);
// int8 codes with one scale a = amax / 127 and the exact fp32 sum per (row, weight
// group): group g is the columns perm[128 g ..] (identity when perm is NULL);
// xs [M][K/128][2] holds the (a, sum) pairs. K % 128 == 0.
hipError_t launch_quantize_groups_sums(const void* x, int x_dtype, const int32_t* perm, int64_t m, int64_t k,
                                       int8_t* q, float* xs, hipStream_t s);
// q [M][K] natural order -> plane order inside each 128-group (element 4u+t of a
// 64-element half-group goes to position 32t + 16*half + u).
hipError_t launch_int8_planes(const int8_t* q, int64_t m, int64_t k, int8_t* q_planes,
                              hipStream_t s);
// q [M][K] -> nibble order for the 4-bit x int8 GEMM (gathered through perm
// when perm is not NULL): inside each 64-element half h of a 128-group, element
// 16t + 8a + 2p + b goes to position 32t + 16h + 4(2a + b) + p.
hipError_t launch_int8_nibbles(const int8_t* q, const int32_t* perm, int64_t m, int64_t k,
                               int8_t* q_nibbles, hipStream_t s);
// x_perm[m][j] = x[m][perm[j]] for 16-bit elements.
hipError_t launch_gather_cols(const uint16_t* x, const int32_t* perm, int64_t m, int64_t k,
                              uint16_t* x_perm, hipStream_t s);

// Decode GEMVs (gemv.hip). Return hipErrorInvalidValue when the staged
// activations do not fit the kernel's LDS budget (caller then routes to GEMM).
bool gemv_t2_fits(int64_t m, int64_t k);
// The complete decode call for one token on ternary weights: fp32, fp16 or
// bf16 activations quantised with the row rule inside the M = 1 GEMV (no
// workspace); M = 1 and K <= 16384.
bool gemv_t2_fused_fits(int64_t m, int64_t k);
hipError_t launch_gemv_t2_fused(const bpw_weights& w, const void* x, int x_dtype, void* y, int y_dtype,
                                hipStream_t s);
// group_scales: x_scale is [M][K/128] (one scale per row and group) instead of
// [M]; only the shapes gemv_t2_group_fits accepts.
bool gemv_t2_group_fits(int64_t m, int64_t k);
// Split-K workspace (fp32 partial slices) the decode GEMV uses for 2 <= M <= 32
// beyond 32 groups with row scales; 0 for other shapes. With less workspace
// than this the long-K kernel runs instead.
size_t gemv_t2_split_bytes(int64_t m, int64_t n, int64_t k, bool group_scales);
hipError_t launch_gemv_t2(const bpw_weights& w, const int8_t* q, const float* x_scale, int64_t m,
                          void* y, int y_dtype, bool group_scales, void* ws, size_t ws_bytes, hipStream_t s);
hipError_t launch_gemv_t2_partials(const bpw_weights& w, const int8_t* q, int64_t m, int64_t m0,
                                   int64_t m1, int64_t n0, int64_t n1, int32_t* out,
                                   hipStream_t s);
// Act order with x in its original column order: the decode kernels gather
// through w.perm themselves (no workspace) at M = 1 and, where M rows of x fit
// in LDS, on the skinny path. Needs 16-byte aligned x and perm.
bool gemv_w4_perm_fits(const bpw_weights& w, int64_t m, const void* x);
hipError_t launch_gemv_w4_perm(const bpw_weights& w, const void* x, int x_dtype, int64_t m, void* y,
                               int y_dtype, hipStream_t s);
bool gemv_w4_fits(int64_t m, int64_t k);
// Bytes of fp32 split-K slices the 4-bit decode needs (2 <= M <= 16 beyond 48
// groups), 0 otherwise; `part` of launch_gemv_w4 must hold that many.
size_t gemv_w4_split_bytes(int64_t m, int64_t n, int64_t k);
hipError_t launch_gemv_w4(const bpw_weights& w, const void* x_sorted, int x_dtype, int64_t m,
                          void* y, int y_dtype, float* part, hipStream_t s);

// Prefill GEMMs (gemm_i8.hip, gemm_w4.hip). x operands already in the order
// the kernels read (int8: plane order; 16-bit: act-order gathered).
hipError_t launch_gemm_t2(const bpw_weights& w, const int8_t* q_planes, const float* x_scale,
                          int64_t m, void* y, int y_dtype, hipStream_t s);
hipError_t launch_gemm_t2_partials(const bpw_weights& w, const int8_t* q_planes, int64_t m,
                                   int64_t m0, int64_t m1, int64_t n0, int64_t n1, int32_t* out,
                                   hipStream_t s);
// 4-bit weights x int8 activations (nibble order), same kernel as the ternary GEMM.
hipError_t launch_gemm_w4a8(const bpw_weights& w, const int8_t* q_nibbles, const float* x_scale,
                            int64_t m, void* y, int y_dtype, hipStream_t s);
hipError_t launch_gemm_w4a8_partials(const bpw_weights& w, const int8_t* q_nibbles, int64_t m,
                                     int64_t m0, int64_t m1, int64_t n0, int64_t n1, int32_t* out,
                                     hipStream_t s);
// Per-(token, group) activation values on the int8 matrix core: ternary weights
// with x_scale [M][G] (q in plane order), or 4-bit weights in the affine form with
// x_scale [M][G][2] = (a, sum) pairs (q in nibble order).
hipError_t launch_gemm_g(const bpw_weights& w, const int8_t* q_ordered, const float* x_scale, int64_t m, void* y,
                         int y_dtype, hipStream_t s);
// Its int32 core: ternary P (code - 1) or 4-bit raw-code dots D.
hipError_t launch_gemm_g_partials(const bpw_weights& w, const int8_t* q_ordered, int64_t m, int64_t m0, int64_t m1,
                                  int64_t n0, int64_t n1, int32_t* out, hipStream_t s);
hipError_t launch_gemm_w4(const bpw_weights& w, const void* x_sorted, int x_dtype, int64_t m,
                          void* y, int y_dtype, hipStream_t s);

// Probes (probe.hip).
int64_t probe_blocks(size_t bytes);
hipError_t launch_probe(int kind, const void* src, void* dst, size_t bytes, hipStream_t s);

}  // namespace bpw
