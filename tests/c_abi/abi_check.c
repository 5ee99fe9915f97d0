/*
 * The C ABI used from C: include/bpw.h compiles as C99 and libbpw.so links and
 * runs its host-only entry points without a GPU.
 *
 * Expected values come from the PQ2 storage format of "Kernel experiments:
 * recorded evidence" (Test 1: a 34-byte block per 128 weights, the fp16 scale
 * first and little-endian, then 32 code bytes holding four 2-bit codes each,
 * first weight in the low bits), written out here by hand, not from the
 * library. Prints "ok" and exits 0 on success; names the failed check and
 * exits 1 otherwise.
 */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "bpw.h"

static int failures = 0;

static void check(int cond, const char* what) {
  if (!cond) {
    printf("FAILED: %s (last error: \"%s\")\n", what, bpw_last_error());
    ++failures;
  }
}

int main(void) {
  enum { N = 2, K = 256, G = K / 128 };
  check(bpw_version() > 0, "bpw_version is positive");

  /* Ternary, fp16 scales: codes K/4 bytes per row, one 2-byte scale per group. */
  bpw_sizes sz;
  check(bpw_packed_sizes(BPW_TERNARY2, BPW_F16, N, K, 128, 0, &sz) == BPW_OK, "packed sizes status");
  check(sz.codes == (size_t)N * K / 4 && sz.scales == (size_t)N * G * 2 && sz.zeros == 0 && sz.perm == 0,
        "ternary plane sizes");

  /* PQ2 blocks: row n, group g has scale bits 0x3C00 + 16 n + g (fp16 around 1.0) and
     code byte j = (n + g + j) % 3 | ((j % 3) << 2) | (1 << 4) | (2 << 6): weights
     4j..4j+3 take codes (n+g+j)%3, j%3, 1, 2. */
  uint8_t src[N][G * 34];
  for (int n = 0; n < N; ++n)
    for (int g = 0; g < G; ++g) {
      uint8_t* b = &src[n][g * 34];
      const uint16_t sbits = (uint16_t)(0x3C00 + 16 * n + g);
      b[0] = (uint8_t)(sbits & 0xFF);
      b[1] = (uint8_t)(sbits >> 8);
      for (int j = 0; j < 32; ++j)
        b[2 + j] = (uint8_t)(((n + g + j) % 3) | ((j % 3) << 2) | (1 << 4) | (2 << 6));
    }
  uint8_t codes[N * K / 4];
  uint16_t scales[N * G];
  memset(codes, 0xAB, sizeof codes);
  memset(scales, 0xAB, sizeof scales);
  check(bpw_prepare_packed(BPW_TERNARY2, BPW_SRC_PQ2_BLOCKS, BPW_F16, N, K, 128, src, NULL, NULL, NULL, codes,
                           scales, NULL, NULL) == BPW_OK,
        "prepare PQ2 blocks");
  int same = 1;
  for (int n = 0; n < N; ++n)
    for (int g = 0; g < G; ++g) {
      same &= memcmp(&codes[n * (K / 4) + g * 32], &src[n][g * 34 + 2], 32) == 0;
      same &= scales[n * G + g] == (uint16_t)(0x3C00 + 16 * n + g);
    }
  check(same, "PQ2 blocks split into code and scale planes");

  /* Refusals, before any launch and without a GPU. */
  check(bpw_prepare_packed(BPW_TERNARY2, BPW_SRC_PQ2_BLOCKS, BPW_F16, N, 200, 128, src, NULL, NULL, NULL, codes,
                           scales, NULL, NULL) == BPW_ESHAPE,
        "K not a multiple of 128 is refused");
  check(strlen(bpw_last_error()) > 0, "a refusal leaves a message");
  check(bpw_packed_sizes(BPW_TERNARY2, BPW_F16, N, K, 128, 0, &sz) == BPW_OK && bpw_last_error()[0] == '\0',
        "success clears the message");

  bpw_weights w;
  memset(&w, 0, sizeof w);
  w.fmt = BPW_TERNARY2;
  w.scale_dtype = BPW_F16;
  w.group = 128;
  w.n = N;
  w.k = 200;
  w.codes = (const void*)(uintptr_t)4096;   /* never dereferenced: validation fails first */
  w.scales = (const void*)(uintptr_t)8192;
  check(bpw_gemv_packed(&w, (const void*)(uintptr_t)65536, BPW_I8, (const float*)(uintptr_t)1024, 1,
                        (void*)(uintptr_t)131072, BPW_F16, NULL, 0, NULL) == BPW_ESHAPE,
        "product with K = 200 is refused");
  w.k = K;
  check(bpw_gemv_packed(&w, (const void*)(uintptr_t)65536, BPW_F16, NULL, 2, (void*)(uintptr_t)131072, BPW_F16,
                        NULL, 0, NULL) == BPW_EUNSUPPORTED,
        "ternary weights with fp16 activations beyond one token are refused by name");
  check(bpw_gemv_packed(&w, (const void*)(uintptr_t)65536, BPW_I32, NULL, 1, (void*)(uintptr_t)131072, BPW_F16,
                        NULL, 0, NULL) == BPW_EUNSUPPORTED,
        "ternary weights with int32 activations are refused by name");

  size_t need = 0;
  check(bpw_workspace_size(&w, 1, BPW_I8, BPW_PATH_GEMV, &need) == BPW_OK && need == 0,
        "the M = 1 ternary GEMV needs no workspace");

  /* 4-bit weights with int8 activations: the GEMM entry, a nibble-ordered copy of q. */
  w.fmt = BPW_INT4_SYM;
  w.scale_dtype = BPW_BF16;
  check(bpw_workspace_size(&w, 64, BPW_I8, BPW_PATH_GEMM, &need) == BPW_OK && need == (size_t)64 * K,
        "the 4-bit x int8 GEMM needs M * K bytes of workspace");
  check(bpw_gemv_packed(&w, (const void*)(uintptr_t)65536, BPW_I8, (const float*)(uintptr_t)1024, 1,
                        (void*)(uintptr_t)131072, BPW_F16, NULL, 0, NULL) == BPW_EUNSUPPORTED,
        "4-bit x int8 through the GEMV entry is refused by name");
  check(bpw_gemm_packed(&w, (const void*)(uintptr_t)65536, BPW_I8, (const float*)(uintptr_t)1024, 64,
                        (void*)(uintptr_t)131072, BPW_F16, NULL, 0, NULL) == BPW_EINVAL,
        "4-bit x int8 without its workspace is refused");

  if (failures) return 1;
  printf("ok\n");
  return 0;
}
