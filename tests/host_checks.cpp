// Host-side checks of libnvfp4's C ABI, built with AddressSanitizer and UndefinedBehaviorSanitizer
// on the host code only (no device code: every call below is rejected, or has nothing to do,
// before any HIP call, so the program needs no GPU).  It drives each entry point's argument
// validation with ordinary mistakes and with sizes at the edges of int64_t, so that an overflow
// in a size computation, an out-of-bounds read of an argument structure or any other undefined
// behaviour in the validation stops the program with the sanitizer's report.
//
// Exit status 0 with "host checks passed" when every expectation holds; 1 with the failing line
// otherwise.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "nvfp4.h"

static int failures = 0;

#define EXPECT(cond)                                                   \
  do {                                                                 \
    if (!(cond)) {                                                     \
      printf("FAILED line %d: %s\n", __LINE__, #cond);                 \
      ++failures;                                                      \
    }                                                                  \
  } while (0)

// Aligned addresses that are never dereferenced: every call that receives them fails
// validation (or has nothing to do) first.
static void *const kFake = (void *)(uintptr_t)0x100000;
static const int64_t kMax = INT64_MAX;
static const int64_t kMax16 = INT64_MAX / 16 * 16;  // largest multiple of 16

static nvfp4_tensor tensor(int64_t rows, int64_t cols, int32_t block_rows) {
  nvfp4_tensor t;
  t.codes = (uint8_t *)kFake;
  t.ld_codes = cols / 2 > 16 ? (cols / 2 + 15) / 16 * 16 : 16;
  t.scales = (uint8_t *)kFake;
  t.ld_scales = cols / 16;
  t.global_scale = (float *)kFake;
  t.rows = rows;
  t.cols = cols;
  t.block_rows = block_rows;
  t.reserved = 0;
  return t;
}

static mxfp4_tensor mxtensor(int64_t rows, int64_t cols) {
  mxfp4_tensor t;
  t.codes = (uint8_t *)kFake;
  t.ld_codes = cols / 2 > 16 ? (cols / 2 + 15) / 16 * 16 : 16;
  t.scales = (uint8_t *)kFake;
  t.ld_scales = cols / 32;
  t.rows = rows;
  t.cols = cols;
  return t;
}

static void status_and_version() {
  for (int s = 0; s < 7; ++s) EXPECT(nvfp4_status_string(s) != NULL);
  EXPECT(nvfp4_status_string(-5) != NULL);
  EXPECT(nvfp4_status_string(1 << 30) != NULL);
  EXPECT(nvfp4_version() >= 100);
}

static void workspace_sizes() {
  EXPECT(nvfp4_quantize_workspace_bytes(8192, 8192) == 8192);
  EXPECT(nvfp4_gemm_workspace_bytes(16, 14336, 4096) >= 8192 + 16 * 2048 + 16 * 256);
  // Sizes no call accepts: the answer saturates instead of wrapping round to a small number.
  EXPECT(nvfp4_gemm_workspace_bytes(kMax, kMax, kMax16) == SIZE_MAX);
  EXPECT(nvfp4_gemm_workspace_bytes((int64_t)1 << 40, 4096, (int64_t)1 << 40) == SIZE_MAX);
  EXPECT(nvfp4_grouped_gemm_workspace_bytes(kMax, kMax16, kMax, 1024) == SIZE_MAX);
  EXPECT(nvfp4_mxfp4_gemm_workspace_bytes(kMax, kMax16) == SIZE_MAX);
  EXPECT(nvfp4_gemm_workspace_bytes(-1, 16, 16) == 8192);
  EXPECT(nvfp4_gemm_workspace_bytes(16, -1, 16) >= 8192);
  EXPECT(nvfp4_mxfp4_gemm_workspace_bytes(-3, 64) == 0);
}

static void quantize_edges() {
  nvfp4_tensor t = tensor(32, 64, 1);
  EXPECT(nvfp4_quantize_1d(NULL, 32, 64, 64, &t, kFake, 8192, NULL) == NVFP4_ERR_NULL);
  EXPECT(nvfp4_quantize_1d(kFake, 32, 64, 64, NULL, kFake, 8192, NULL) == NVFP4_ERR_NULL);
  // Huge and negative sizes, with an output descriptor that claims the same sizes.
  const int64_t sizes[][3] = {{kMax, kMax16, kMax16},  {kMax16, 16, 16},  {1, kMax16, kMax16},
                              {(int64_t)1 << 40, (int64_t)1 << 40, (int64_t)1 << 40},
                              {-1, 64, 64},            {32, -16, 64},     {32, 64, -64},
                              {INT64_MIN, 64, 64},     {32, 64, INT64_MIN / 16 * 16}};
  for (const auto &s : sizes) {
    nvfp4_tensor o = tensor(s[0], s[1], 1);
    EXPECT(nvfp4_quantize_1d(kFake, s[0], s[1], s[2], &o, kFake, 8192, NULL) != NVFP4_OK);
    nvfp4_tensor o2 = tensor(s[0], s[1], 16);
    EXPECT(nvfp4_quantize_2d(kFake, s[0], s[1], s[2], &o2, kFake, 8192, NULL) != NVFP4_OK);
    EXPECT(nvfp4_quantize_mse(kFake, s[0], s[1], s[2], &o2, kFake, 8192, NULL) != NVFP4_OK);
    EXPECT(nvfp4_dequantize(&o, kFake, s[2], NVFP4_OUT_F32, NULL) != NVFP4_OK);
  }
  // Leading dimensions near the top of the range.
  nvfp4_tensor big_ld = tensor(32, 64, 1);
  big_ld.ld_codes = kMax16;
  big_ld.ld_scales = kMax;
  EXPECT(nvfp4_dequantize(&big_ld, kFake, kMax16, NVFP4_OUT_F32, NULL) != NVFP4_OK);
  EXPECT(nvfp4_quantize_1d(kFake, 32, 64, kMax16, &big_ld, kFake, 8192, NULL) != NVFP4_OK);
  // Empty tensors: nothing to do, no buffers needed.
  nvfp4_tensor e = tensor(0, 64, 1);
  e.codes = NULL;
  e.scales = NULL;
  e.global_scale = NULL;
  EXPECT(nvfp4_quantize_1d(NULL, 0, 64, 64, &e, NULL, 0, NULL) == NVFP4_OK);
  EXPECT(nvfp4_dequantize(&e, NULL, 64, NVFP4_OUT_BF16, NULL) == NVFP4_OK);
}

static void gemm_edges() {
  nvfp4_tensor w = tensor(128, 256, 16);
  EXPECT(nvfp4_gemm_w4a4(kFake, 64, 256, 256, NULL, NULL, kFake, 128, kFake, 1 << 30, NULL) ==
         NVFP4_ERR_NULL);
  EXPECT(nvfp4_gemm_w4a4(kFake, 64, 240, 240, NULL, &w, kFake, 128, kFake, 1 << 30, NULL) ==
         NVFP4_ERR_SHAPE);
  // A quantized operand that claims enormous K: rejected, and the workspace size it would need
  // is not computed with a wrapped product.
  const int64_t ks[] = {kMax16, (int64_t)1 << 40, (int64_t)1 << 32};
  for (int64_t k : ks) {
    nvfp4_tensor wk = tensor(128, k, 16);
    nvfp4_tensor ak = tensor(64, k, 1);
    EXPECT(nvfp4_gemm_w4a4(NULL, 64, k, 0, &ak, &wk, kFake, 128, kFake, 1 << 30, NULL) !=
           NVFP4_OK);
    EXPECT(nvfp4_gemm_w4a4(kFake, 64, k, k, NULL, &wk, kFake, 128, kFake, 1 << 30, NULL) !=
           NVFP4_OK);
    EXPECT(nvfp4_gemm_w4a4_noalloc(NULL, 64, k, 0, &ak, &wk, kFake, 128, NULL) != NVFP4_OK);
    EXPECT(nvfp4_gemm_w4a16(kFake, 8, k, k, &wk, kFake, 128, NULL) != NVFP4_OK);
  }
  // Huge M and N.
  nvfp4_tensor wn = tensor(kMax16, 256, 16);
  EXPECT(nvfp4_gemm_w4a4(kFake, 64, 256, 256, NULL, &wn, kFake, kMax, kFake, SIZE_MAX, NULL) !=
         NVFP4_OK);
  EXPECT(nvfp4_gemm_w4a4(kFake, kMax, 256, 256, NULL, &w, kFake, 128, kFake, SIZE_MAX, NULL) !=
         NVFP4_OK);
  EXPECT(nvfp4_gemm_w4a4_noalloc(kFake, kMax, 256, 256, NULL, &w, kFake, 128, NULL) != NVFP4_OK);
  EXPECT(nvfp4_gemm_w4a16(kFake, kMax, 256, 256, &w, kFake, 128, NULL) != NVFP4_OK);
  EXPECT(nvfp4_gemm_w4a16(kFake, 8, 256, 256, &wn, kFake, kMax, NULL) != NVFP4_OK);
  // Empty products.
  EXPECT(nvfp4_gemm_w4a4(NULL, 0, 256, 0, NULL, &w, NULL, 128, NULL, 0, NULL) == NVFP4_OK);
  EXPECT(nvfp4_gemm_w4a16(NULL, 0, 256, 0, &w, NULL, 128, NULL) == NVFP4_OK);
}

static void grouped_edges() {
  nvfp4_tensor w = tensor(8 * 64, 128, 16);
  const int32_t *idx = (const int32_t *)kFake;
  EXPECT(nvfp4_grouped_gemm_w4a4(kFake, 32, 128, 128, NULL, idx, 64, idx, 0, &w, 64, kFake, 64,
                                 kFake, 1 << 30, NULL) == NVFP4_ERR_SHAPE);
  EXPECT(nvfp4_grouped_gemm_w4a4(kFake, 32, 128, 128, NULL, idx, 64, idx, -7, &w, 64, kFake, 64,
                                 kFake, 1 << 30, NULL) == NVFP4_ERR_SHAPE);
  // Expert width so large that num_groups * n leaves int64_t.
  nvfp4_tensor wn = tensor(kMax16, 128, 16);
  EXPECT(nvfp4_grouped_gemm_w4a4(kFake, 32, 128, 128, NULL, idx, 64, idx, 1024, &wn, kMax16,
                                 kFake, kMax, kFake, SIZE_MAX, NULL) != NVFP4_OK);
  EXPECT(nvfp4_grouped_gemm_w4a4(kFake, 32, 128, 128, NULL, idx, 64, idx, 8, &wn,
                                 kMax / 8 / 16 * 16 + 16, kFake, kMax, kFake, SIZE_MAX,
                                 NULL) != NVFP4_OK);
  // Huge token and row counts, and huge K.
  EXPECT(nvfp4_grouped_gemm_w4a4(kFake, kMax, 128, 128, NULL, idx, kMax, idx, 8, &w, 64, kFake,
                                 64, kFake, SIZE_MAX, NULL) != NVFP4_OK);
  nvfp4_tensor wk = tensor(8 * 64, kMax16, 16);
  nvfp4_tensor ak = tensor(32, kMax16, 1);
  EXPECT(nvfp4_grouped_gemm_w4a4(NULL, 32, kMax16, 0, &ak, idx, 64, idx, 8, &wk, 64, kFake, 64,
                                 kFake, SIZE_MAX, NULL) != NVFP4_OK);
  EXPECT(nvfp4_grouped_gemm_w4a4(NULL, 4, 128, 128, NULL, NULL, 0, NULL, 2, &w, 64, NULL, 64,
                                 NULL, 0, NULL) == NVFP4_OK);
}

static void mxfp4_edges() {
  const int64_t sizes[][3] = {{kMax, kMax / 32 * 32, kMax16}, {(int64_t)1 << 40, 1 << 20, 1 << 20},
                              {-1, 64, 64}, {32, -32, 64}};
  for (const auto &s : sizes) {
    mxfp4_tensor q = mxtensor(s[0], s[1]);
    EXPECT(nvfp4_mxfp4_quantize(kFake, s[0], s[1], s[2], &q, NULL) != NVFP4_OK);
    EXPECT(nvfp4_mxfp4_dequantize(&q, kFake, s[2], NVFP4_OUT_F32, NULL) != NVFP4_OK);
  }
  mxfp4_tensor w = mxtensor(128, 256);
  mxfp4_tensor wk = mxtensor(128, kMax / 32 * 32);
  mxfp4_tensor ak = mxtensor(8, kMax / 32 * 32);
  EXPECT(nvfp4_mxfp4_gemm(NULL, 8, kMax / 32 * 32, 0, &ak, &wk, kFake, 128, NULL, 0, NULL) !=
         NVFP4_OK);
  EXPECT(nvfp4_mxfp4_gemm(kFake, kMax, 256, 256, NULL, &w, kFake, 128, kFake, SIZE_MAX, NULL) !=
         NVFP4_OK);
  EXPECT(nvfp4_mxfp4_gemm(NULL, 0, 256, 0, NULL, &w, NULL, 128, NULL, 0, NULL) == NVFP4_OK);
}

int main() {
  setvbuf(stdout, NULL, _IONBF, 0);  // a sanitizer stop must not swallow earlier lines
  status_and_version();
  workspace_sizes();
  quantize_edges();
  gemm_edges();
  grouped_edges();
  mxfp4_edges();
  if (failures) {
    printf("%d host check(s) failed\n", failures);
    return 1;
  }
  printf("host checks passed\n");
  return 0;
}
