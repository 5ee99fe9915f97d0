/*
 * bpw.h -- C ABI of the bit-packed weight library (AMD Instinct MI355X, gfx950).
 *
 * Computes y = x @ W^T for a weight matrix W [N, K] stored group-quantised:
 * 2-bit ternary codes or 4-bit codes, one fp16/bf16 scale (and optionally one
 * 4-bit zero point) per group of 128 along K, with an optional act-order
 * permutation of K. Activations are fp16/bf16, or int8 with one fp32 scale per
 * row (or, for the decode GEMV, per row and 128-group). Sources: "Kernel experiments: recorded evidence" (ternary PQ2 format,
 * section A and Tests 1, 2, 6-8, 21), "mate: Marlin-class W4A16 GEMM for
 * mp_31 (SQMMA int4 x fp16) - #6" (4-bit codes, zero points, act order) and
 * "TensorFold PR #1176" (4-bit weights against int8 activations on the int8
 * matrix instruction).
 *
 * Conventions for every entry point (the shape of the pages' own interfaces:
 * "Kernel experiments", Test 1's prepare step validates its input and raises
 * naming the violated condition before any work, and Test 23's launcher takes
 * caller-allocated buffers, the current stream and returns an int status):
 *  - "host" pointers are ordinary CPU memory; "device" pointers are GPU memory
 *    owned by the caller (e.g. allocated through PyTorch). The library never
 *    allocates or frees device memory and never synchronises a stream, except
 *    where an entry point says otherwise.
 *  - Work is launched only on the HIP stream passed in (NULL = default stream).
 *  - Matrices are dense row-major. Device planes must be 16-byte aligned.
 *  - Every argument is validated before anything is launched. On failure the
 *    call returns a nonzero status, touches no output, and bpw_last_error()
 *    (thread-local) names the violated invariant. A launch failure returns
 *    BPW_EHIP; faults inside a kernel surface at the caller's next sync.
 *  - Results are bit-identical from run to run (no atomics, fixed-order sums).
 */
#ifndef BPW_H_
#define BPW_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ---------------------------------------------------- */
#define BPW_OK 0
#define BPW_EINVAL 1        /* NULL pointer, unknown enum value, negative size   */
#define BPW_ESHAPE 2        /* inconsistent sizes (K % 128, window, buffer size) */
#define BPW_EALIGN 3        /* pointer not aligned as required                   */
#define BPW_EGIDX 4         /* act-order g_idx malformed                          */
#define BPW_EUNSUPPORTED 5  /* valid request this library does not implement     */
#define BPW_EHIP 6          /* HIP runtime reported an error                      */

/* ---- weight formats -------------------------------------------------- */
#define BPW_TERNARY2 1 /* 2-bit codes, value = code - 1 (code 3 decodes to +2); fp16 scales */
#define BPW_INT4_SYM 2 /* 4-bit codes, value = code - 8                                     */
#define BPW_INT4_ZP 3  /* 4-bit codes, value = code - zero[n, group]                        */

/* ---- element types --------------------------------------------------- */
#define BPW_F32 0
#define BPW_F16 1
#define BPW_BF16 2
#define BPW_I8 3
#define BPW_I32 4
/* int8 activations with one fp32 scale per (row, 128-group): x_scale [M][K/128].
 * Accepted by bpw_gemv_packed for ternary weights ("Kernel experiments",
 * Test 6: the quantiser's scale is per group of 128 activations). */
#define BPW_I8G 5
/* int8 activations with, per (row, weight group), one fp32 scale a and the
 * exact fp32 sum of the unquantised activations: x_scale [M][K/128][2] holding
 * (a, sum) pairs, as written by bpw_quantize_groups_sums. Accepted by
 * bpw_gemm_packed for 4-bit weights ("TensorFold PR #1176", "What changes":
 * the int8 prompt GEMM takes s * a * (code . q) + b * sum(x) per group). */
#define BPW_I8GS 6

/* ---- source layouts accepted by bpw_prepare_packed ------------------- */
#define BPW_SRC_PQ2_BLOCKS 1 /* ternary only: [N][G][34] = fp16 scale (little-endian) + 32 code bytes */
#define BPW_SRC_PLANES 2     /* packed code plane (layout below) + scales [N][G] (+ zero plane)      */
#define BPW_SRC_CODES_U8 3   /* one code per byte [N][K] + scales [N][G] (+ zeros one per byte [N][G]) */

/* ---- partial-sum cores for bpw_partials ------------------------------ */
#define BPW_PATH_GEMV 0
#define BPW_PATH_GEMM 1
#define BPW_PATH_GEMM_RAW 2 /* bpw_partials only: raw-code dots of the I8GS GEMM core */

/* ---- HBM probes for bpw_probe ---------------------------------------- */
#define BPW_PROBE_READ 0 /* read every byte of src (16-byte loads), write one word per block to dst */
#define BPW_PROBE_COPY 1 /* copy bytes from src to dst (16-byte loads and stores)                   */

/*
 * Prepared (device) weight layout, "separate planes": one code plane, one
 * scale plane, optionally one zero-point plane and one permutation.
 *  codes  : TERNARY2  uint8 [N][K/4]; in each row, byte 32g+j holds weights
 *                     128g+4j+t at bits 2t..2t+1 (t = 0..3).
 *           INT4_*    uint8 [N][K/2]; byte b holds weight 2b in the low
 *                     nibble and 2b+1 in the high nibble.
 *  scales : [N][G] of scale_dtype (G = K/128).
 *  zeros  : INT4_ZP only: uint8 [N][ceil(G/2)]; group 2i in the low nibble,
 *           2i+1 in the high nibble. NULL otherwise.
 *  perm   : act-order only: int32 [K]; column j of the prepared planes is
 *           column perm[j] of the original weight, so group j/128 of the
 *           planes is contiguous. NULL when the weight has no act order.
 * With act order, y = x[:, perm] @ W_prepared^T, which equals x @ W^T.
 */
typedef struct bpw_weights {
  int32_t fmt;         /* BPW_TERNARY2 | BPW_INT4_SYM | BPW_INT4_ZP          */
  int32_t scale_dtype; /* BPW_F16 | BPW_BF16 (TERNARY2: BPW_F16 only)        */
  int32_t group;       /* 128                                                */
  int32_t reserved;    /* must be 0                                          */
  int64_t n;           /* output features (rows of W), >= 1                  */
  int64_t k;           /* input features, a positive multiple of 128         */
  const void* codes;   /* device                                             */
  const void* scales;  /* device                                             */
  const void* zeros;   /* device or NULL                                     */
  const int32_t* perm; /* device or NULL                                     */
} bpw_weights;

typedef struct bpw_sizes {
  size_t codes, scales, zeros, perm; /* bytes of each prepared plane (0 = absent) */
} bpw_sizes;

/* Library version (major * 10000 + minor * 100 + patch); library metadata,
 * not from the pages. */
int bpw_version(void);

/* Thread-local text of the last error of this thread ("" after success): the
 * text names the violated invariant, as the pages' prepare and launch steps
 * do in their exceptions ("Kernel experiments", Tests 1 and 23). */
const char* bpw_last_error(void);

/*
 * Byte sizes of the prepared planes for an N x K weight of format fmt
 * ("Kernel experiments", Test 1: separate code and scale buffers keep exactly
 * 34 bytes per 128-weight block, 32 of codes and a 2-byte scale; the mate PR's
 * 4-bit codes add half a byte per weight, a zero-point nibble per group and,
 * with act order, the K-entry permutation). scale_dtype (F16 or BF16) sets
 * the scale plane's element size; the zero plane is present for INT4_ZP.
 * Logical weight bytes per product = codes + scales + zeros (the perm plane is
 * K int32 and is read once per call, not per row). Host only; never touches
 * the GPU.
 */
int bpw_packed_sizes(int fmt, int scale_dtype, int64_t n, int64_t k, int group, int has_perm,
                     bpw_sizes* out);

/*
 * Repack user weights into the prepared planes (one-time, host only, no GPU).
 * Source: "Kernel experiments", Test 1 (prepare_pq2 splits 34-byte blocks into
 * code and scale planes, with the same 34 bytes per 128 weights) and the mate
 * PR's "Act order" section (sort K by group, keep the permutation, refuse a
 * g_idx whose sorted groups are not runs of exactly 128).
 *  src_codes  host, layout per src_format:
 *               PQ2_BLOCKS [N][G*34] (ternary; src_scales must be NULL),
 *               PLANES     the prepared code layout above (original K order),
 *               CODES_U8   [N][K] one code per byte (0..3 ternary, 0..15 int4).
 *  src_scales host [N][G] of scale_dtype (NULL for PQ2_BLOCKS).
 *  src_zeros  host, INT4_ZP only: PLANES -> [N][ceil(G/2)] nibbles (low = even
 *             group), CODES_U8 -> [N][G] one per byte. NULL otherwise.
 *  g_idx      host int32 [K] group of each original column, or NULL (no act
 *             order). Every group id must be in 0..G-1 and own exactly 128
 *             columns, else BPW_EGIDX naming the group and its count.
 *  dst_*      host buffers sized by bpw_packed_sizes (dst_zeros NULL unless
 *             INT4_ZP, dst_perm NULL unless g_idx). perm = stable argsort(g_idx).
 * Codes out of range (ternary > 3, int4 > 15 in CODES_U8) return BPW_EINVAL.
 */
int bpw_prepare_packed(int fmt, int src_format, int scale_dtype, int64_t n, int64_t k, int group,
                       const void* src_codes, const void* src_scales, const uint8_t* src_zeros,
                       const int32_t* g_idx, void* dst_codes, void* dst_scales, void* dst_zeros,
                       int32_t* dst_perm);

/*
 * int8 activation quantiser, one scale per row. Source: "Kernel experiments",
 * Test 6 (group-128 quantiser) and Test 8 (the fp32 reciprocal-multiply scale):
 *   scale[m] = fl32(max_k |x[m,k]| * fl32(1/127)),
 *   q[m,k]   = clamp(round_half_even(x[m,k] / (scale[m] > 0 ? scale[m] : 1)), -127, 127)
 * with an IEEE fp32 division. A row holding a NaN or an infinity gets
 * x_scale NaN and all-zero codes, so every product output of that row is NaN
 * (the pages say nothing of such inputs; this makes them visible).
 * x: device [M][K] of x_dtype (F32/F16/BF16);
 * q: device int8 [M][K]; x_scale: device fp32 [M]. K >= 1, no multiple needed.
 */
int bpw_quantize_rows(const void* x, int x_dtype, int64_t m, int64_t k, int8_t* q, float* x_scale,
                      void* stream);

/*
 * int8 activation quantiser, one scale per (row, 128-group), the same rule
 * with the group's own max ("Kernel experiments", Test 6, group-128 form):
 *   scale[m,g] = fl32(max_{k in g} |x[m,k]| * fl32(1/127)),
 *   q[m,k]     = clamp(round_half_even(x[m,k] / (scale[m,g] > 0 ? scale[m,g] : 1)), -127, 127).
 * A group holding a NaN or an infinity gets scale NaN and zero codes, as for rows.
 * x: device [M][K] of x_dtype (F32/F16/BF16); K a multiple of 128.
 * q: device int8 [M][K], 16-byte aligned; x_scale: device fp32 [M][K/128].
 */
int bpw_quantize_groups(const void* x, int x_dtype, int64_t m, int64_t k, int8_t* q, float* x_scale,
                        void* stream);

/*
 * int8 activation quantiser of the 4-bit x int8 prefill in its affine form
 * ("TensorFold PR #1176", "What changes": tf_w4a8_quantize writes each
 * activation group as int8 codes with one fp32 scale a = amax / 127 and the
 * group's exact fp32 sum). Here a group is one weight group: the 128 columns
 * perm[128 g .. 128 g + 127] of a row (columns 128 g .. when perm is NULL), so
 * that a and the sum pair with the weight's scale and zero point of group g.
 *   a[m,g]   = fl32(max_{k in g} |x[m,k]| / 127)            (IEEE division)
 *   q[m,k]   = clamp(round_half_even(x[m,k] / (a > 0 ? a : 1)), -127, 127)
 *   sum[m,g] = the exact sum of x[m,k] over the group, rounded once to fp32
 *              (exact whenever the group's nonzero values span at most 2^73
 *              in magnitude, always for fp16 inputs)
 * A group holding a NaN or an infinity gets a = sum = NaN and zero codes.
 * x: device [M][K] of x_dtype (F32/F16/BF16), K a multiple of 128;
 * perm: device int32 [K] (the prepared weight's perm) or NULL; entries outside
 *   [0, K) are read as zero and their codes are not written;
 * q: device int8 [M][K], codes in the columns of x, 16-byte aligned;
 * x_scale_sum: device fp32 [M][K/128][2], (a, sum) pairs, 8-byte aligned.
 */
int bpw_quantize_groups_sums(const void* x, int x_dtype, int64_t m, int64_t k, const int32_t* perm, int8_t* q,
                             float* x_scale_sum, void* stream);

/*
 * Device workspace (bytes, 256-byte aligned start) that bpw_gemv_packed /
 * bpw_gemm_packed need for this weight, M and activation type; 0 if none.
 * The caller allocates it, as the pages' launchers allocate their intermediate
 * buffers before the launch ("Kernel experiments", Test 23: the quantised
 * fragments and, when K is split, the fp32 partial buffer [split][M][N]).
 * entry: BPW_PATH_GEMV or BPW_PATH_GEMM. Host only.
 */
int bpw_workspace_size(const bpw_weights* w, int64_t m, int x_dtype, int entry, size_t* bytes);

/*
 * y = x @ W^T, decode-shaped (tuned for M <= 16; any M >= 1 accepted): the
 * pages' GEMV, with W the dequantised weight of the prepared planes
 * ("Kernel experiments", Test 6: per 128-group an exact integer dot of int8
 * activations with the ternary values, folded with the activation and weight
 * scales; the mate PR: int4 codes minus zero points times the group scale,
 * against fp16/bf16 activations, with act order).
 * Supported (fmt, x_dtype): TERNARY2 x I8 (x_scale device fp32 [M] required),
 * TERNARY2 x I8G (x_scale device fp32 [M][K/128]; M <= 32, larger M and the
 * GEMM entry return BPW_EUNSUPPORTED), INT4_SYM / INT4_ZP x F16 or BF16
 * (scale_dtype == x_dtype, x_scale NULL). INT4_SYM / INT4_ZP x I8 (either
 * scale dtype, x_scale device fp32 [M]) runs through bpw_gemm_packed only
 * (here BPW_EUNSUPPORTED). TERNARY2 x F32, F16 or BF16 (x_scale NULL) is the
 * complete decode call for one token: M = 1 and K <= 16384 only (other shapes
 * BPW_EUNSUPPORTED; quantise with bpw_quantize_rows first), no workspace. The
 * row is quantised with bpw_quantize_rows' rule inside the GEMV launch, and
 * y is bit for bit what bpw_quantize_rows followed by the TERNARY2 x I8 call
 * gives ("Kernel experiments", Test 6: the activation quantiser is part of
 * the timed decode call; Test 18).
 * Anything else returns BPW_EUNSUPPORTED. y: device [M][N] of y_dtype
 * (F32, F16 or BF16; round-to-nearest-even from fp32).
 * Numerics: int8 -> exact int32 group partials, fp32 fold
 * y = x_scale[m] * sum_g scale[n,g] * P[m,n,g] (I8G: y = sum_g x_scale[m,g] *
 * scale[n,g] * P[m,n,g], the two scales multiplied in fp32 first). 4-bit -> the group partial
 * sum_k x * (code - zero) is accumulated in fp32 from exact products and the
 * group scale is applied to it (the weight is never rounded).
 * workspace: device, at least bpw_workspace_size(..., BPW_PATH_GEMV) bytes, or
 * NULL when that size is 0. M <= 32 runs the decode kernels; larger M is routed
 * to the bpw_gemm_packed kernels (and takes their numerics).
 * Split-K (ternary x I8, 2 <= M <= 32, K > 4096): K is cut into slices of 32
 * groups computed side by side; the workspace holds their fp32 sums
 * [slices][M][N], added in slice order by a second launch on the same stream
 * (deterministic). "Kernel experiments: recorded evidence", Test 21: split-K
 * gives the small-output down projection more blocks, and a second kernel adds
 * the partial sums in a fixed order; Test 30: split-K for small-output shapes.
 * The same for INT4_SYM / INT4_ZP x F16 / BF16 with 2 <= M <= 16 and more than
 * 48 groups (slices of at most 16 groups); with act order the workspace holds
 * the gathered activations first, then the slices. At M = 1 a 4-bit K longer
 * than 8192 is split over the waves of one workgroup instead (no workspace;
 * the mate PR splits K of its small-M kernel with fp32 partials and a fixed
 * reduction order).
 */
int bpw_gemv_packed(const bpw_weights* w, const void* x, int x_dtype, const float* x_scale,
                    int64_t m, void* y, int y_dtype, void* workspace, size_t workspace_bytes,
                    void* stream);

/*
 * bpw_gemv_packed for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same product, kernels and results, with no workspace argument. The
 * workspace comes from a fixed array of BPW_SCRATCH_BYTES in this library's
 * device memory, one per GPU, held until the process ends; this call never
 * allocates or frees. A call whose workspace (bpw_workspace_size with
 * BPW_PATH_GEMV) exceeds BPW_SCRATCH_BYTES returns BPW_ESHAPE before any
 * launch. Every call on one GPU shares that GPU's array and it keeps the last
 * call's contents (no call reads bytes it did not write first): calls that
 * overlap on one GPU (several streams or threads) race and must be ordered by
 * the caller.
 */
#define BPW_SCRATCH_BYTES (16 << 20)
int bpw_gemv_packed_scratch(const bpw_weights* w, const void* x, int x_dtype, const float* x_scale,
                            int64_t m, void* y, int y_dtype, void* stream);

/*
 * y = x @ W^T, prefill-shaped (large M). Same arguments and combinations as
 * bpw_gemv_packed, plus 4-bit weights x I8 or I8GS.
 * Numerics: ternary x int8 -> as above (int8 MFMA, exact int32 group
 * partials). 4-bit x F16/BF16 -> each weight is dequantised to the activation dtype,
 * round-to-nearest-even of (code - zero) * scale, then multiplied on MFMA with
 * fp32 accumulation (the float path of the mate PR: unpack int4 to the
 * activation type before the matrix instruction).
 * 4-bit x I8 ("TensorFold PR #1176", the int8 prompt GEMM: a 4-bit code is an
 * exact int8, so the group dot runs exactly on the int8 matrix instruction),
 * with one activation scale per row:
 * P[m,n,g] = sum_{k in g} q[m,k] * (code[n,k] - zero[n,g]) in exact int32
 * (zero 8 for INT4_SYM), then y = x_scale[m] * sum_g scale[n,g] * P[m,n,g] in
 * fp32. With act order, q is gathered through perm. Needs a workspace of
 * M * K bytes (a reordered copy of q).
 * 4-bit x I8GS (the same page's affine form, its own formula): with
 * b[n,g] = -zero[n,g] * scale[n,g] (zero 8 for INT4_SYM),
 *   D[m,n,g] = sum_{k in g} q[m,k] * code[n,k]   (raw codes 0..15, exact int32)
 *   y[m,n]   = sum_g scale[n,g] * a[m,g] * D[m,n,g] + b[n,g] * sum[m,g]   (fp32)
 * where (a, sum) = x_scale[m][g][0..1] from bpw_quantize_groups_sums run with
 * the weight's perm. Each group's int32 D is converted exactly to fp32 and
 * folded as scale * fma(D, a, -8 * sum) (symmetric codes) or
 * scale * (D * a) + b * sum (zero points). Needs a workspace of M * K bytes.
 * Ternary x I8G (one activation scale per (row, 128-group), "Kernel
 * experiments", Test 7's fold partial * x_scale * w_scale per group):
 * y = sum_g x_scale[m,g] * scale[n,g] * P[m,n,g]; workspace M * K bytes.
 * Ternary x F32 / F16 / BF16 (the one-token complete call) runs through
 * bpw_gemv_packed only (here BPW_EUNSUPPORTED).
 */
int bpw_gemm_packed(const bpw_weights* w, const void* x, int x_dtype, const float* x_scale,
                    int64_t m, void* y, int y_dtype, void* workspace, size_t workspace_bytes,
                    void* stream);

/*
 * Verification only: exact int32 group partials
 *   out[(m-m0)][(n-n0)][g] = sum_{k in group g} q[m,k] * value(n,k)
 * for m0 <= m < m1, n0 <= n < n1, computed by the same kernel core as the
 * product, with value = code - 1 (TERNARY2) or code - zero (INT4_*; group g
 * in act order, q gathered through perm). Path BPW_PATH_GEMV: TERNARY2 and
 * M <= 32 only; BPW_PATH_GEMM: any format and M; BPW_PATH_GEMM_RAW: INT4_*
 * only, value = code (the raw-code dots D of the I8GS product, from its
 * kernel). q: device int8 [M][K].
 * out: device int32 [(m1-m0)][(n1-n0)][G]. workspace as for the product.
 */
int bpw_partials(const bpw_weights* w, const int8_t* q, int64_t m, int path, int64_t m0,
                 int64_t m1, int64_t n0, int64_t n1, int32_t* out, void* workspace,
                 size_t workspace_bytes, void* stream);

/*
 * Memory-system probe ("Kernel experiments", Test 24: bandwidth probes that
 * only load, to separate the access pattern from the arithmetic), used to
 * calibrate byte counters and as the streaming ceiling: BPW_PROBE_READ reads
 * `bytes` from src (device, 16-byte aligned, bytes % 16 == 0) and writes one
 * uint32 per workgroup into dst (device, at least bpw_probe_blocks(bytes) * 4
 * bytes); BPW_PROBE_COPY copies `bytes` from src to dst.
 */
int bpw_probe(int kind, const void* src, void* dst, size_t bytes, void* stream);
int64_t bpw_probe_blocks(size_t bytes);

#ifdef __cplusplus
}
#endif

#endif /* BPW_H_ */
