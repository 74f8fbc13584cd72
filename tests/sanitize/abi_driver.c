/* Calls every entry point of include/nvfp4.h with arguments its host-side
 * validation must reject (and a few that need no launch), for a run of the
 * library's host code under AddressSanitizer and UndefinedBehaviorSanitizer on
 * the CPU.  No GPU is touched: every call returns before its first launch.
 * Written in C, the language of the ABI: a C caller may pass any int where an
 * enum is declared, and the library must reject it without undefined
 * behaviour. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "nvfp4.h"

static int failures = 0;
#define EXPECT(cond)                                               \
  do {                                                             \
    if (!(cond)) {                                                 \
      fprintf(stderr, "failed: %s (line %d)\n", #cond, __LINE__); \
      ++failures;                                                  \
    }                                                              \
  } while (0)

int main(void) {
  void* F = (void*)(uintptr_t)0x10000;  /* aligned, never dereferenced */
  void* U = (void*)(uintptr_t)0x10004;  /* misaligned */
  uint8_t* F8 = ((uint8_t*)(F));
  float* Ff = ((float*)(F));
  nvfp4_config cfg;
  memset(&cfg, 0, sizeof cfg);
  cfg.block = NVFP4_BLOCK_1D;
  cfg.emit_rowwise = 1;
  cfg.rule = NVFP4_RULE_NONE;
  cfg.scale_cap = 448.0f;
  nvfp4_outputs out = {F8, F8, F8, F8, Ff};

  EXPECT(nvfp4_abi_version() == NVFP4_ABI_VERSION);
  for (int s = -1; s < 10; ++s) EXPECT(nvfp4_status_string((nvfp4_status)s) != NULL);
  (void)nvfp4_rht_signs_from_seed(0xFFFFFFFFFFFFFFFFull);
  EXPECT(nvfp4_amax_workspace_bytes(-1, 5) == 0);
  EXPECT(nvfp4_amax_workspace_bytes(1ll << 29, 1ll << 29) > 0);
  EXPECT(nvfp4_amax_workspace_bytes(1ll << 40, 1ll << 40) == 0);

  /* amax */
  const size_t ws = nvfp4_amax_workspace_bytes(64, 64);
  EXPECT(nvfp4_amax(F, NVFP4_IN_BF16, -1, 64, &cfg, Ff, F, ws, NULL) == NVFP4_ERR_SHAPE);
  EXPECT(nvfp4_amax(F, (nvfp4_dtype)(9), 64, 64, &cfg, Ff, F, ws, NULL) == NVFP4_ERR_DTYPE);
  EXPECT(nvfp4_amax(F, NVFP4_IN_BF16, 64, 64, &cfg, NULL, F, ws, NULL) == NVFP4_ERR_NULL);
  EXPECT(nvfp4_amax(NULL, NVFP4_IN_BF16, 64, 64, &cfg, Ff, F, ws, NULL) == NVFP4_ERR_NULL);
  EXPECT(nvfp4_amax(U, NVFP4_IN_BF16, 64, 64, &cfg, Ff, F, ws, NULL) == NVFP4_ERR_ALIGN);
  EXPECT(nvfp4_amax(F, NVFP4_IN_BF16, 64, 64, &cfg, Ff, F, ws - 1, NULL) == NVFP4_ERR_WORKSPACE);
  EXPECT(nvfp4_amax(F, NVFP4_IN_BF16, 64, 64, &cfg, Ff, NULL, ws, NULL) == NVFP4_ERR_WORKSPACE);
  cfg.rht = 1;
  EXPECT(nvfp4_amax(F, NVFP4_IN_BF16, 64, 24, &cfg, Ff, F, ws, NULL) == NVFP4_ERR_SHAPE);
  cfg.rht = 0;

  /* quantize */
  EXPECT(nvfp4_quantize(F, NVFP4_IN_BF16, 64, 64, NULL, Ff, &out, NULL) == NVFP4_ERR_NULL);
  EXPECT(nvfp4_quantize(F, NVFP4_IN_BF16, 64, 64, &cfg, NULL, &out, NULL) == NVFP4_ERR_NULL);
  EXPECT(nvfp4_quantize(F, NVFP4_IN_BF16, 64, 24, &cfg, Ff, &out, NULL) == NVFP4_ERR_SHAPE);
  EXPECT(nvfp4_quantize(F, NVFP4_IN_BF16, -16, 64, &cfg, Ff, &out, NULL) == NVFP4_ERR_SHAPE);
  EXPECT(nvfp4_quantize(U, NVFP4_IN_BF16, 64, 64, &cfg, Ff, &out, NULL) == NVFP4_ERR_ALIGN);
  EXPECT(nvfp4_quantize(F, (nvfp4_dtype)(-3), 64, 64, &cfg, Ff, &out, NULL) == NVFP4_ERR_DTYPE);
  nvfp4_config c2 = cfg;
  c2.scale_cap = 300.0f;
  EXPECT(nvfp4_quantize(F, NVFP4_IN_BF16, 64, 64, &c2, Ff, &out, NULL) == NVFP4_ERR_UNSUPPORTED);
  c2 = cfg;
  c2.rule = 17;
  EXPECT(nvfp4_quantize(F, NVFP4_IN_BF16, 64, 64, &c2, Ff, &out, NULL) == NVFP4_ERR_UNSUPPORTED);
  c2 = cfg;
  c2.block = 5;
  EXPECT(nvfp4_quantize(F, NVFP4_IN_BF16, 64, 64, &c2, Ff, &out, NULL) == NVFP4_ERR_UNSUPPORTED);
  c2 = cfg;
  c2.emit_colwise = 1;
  EXPECT(nvfp4_quantize(F, NVFP4_IN_BF16, 24, 64, &c2, Ff, &out, NULL) == NVFP4_ERR_SHAPE);
  EXPECT(nvfp4_quantize(F, NVFP4_IN_BF16, 16, (1ll << 24) + 16, &c2, Ff, &out, NULL) == NVFP4_ERR_SHAPE);
  c2.rht = 1;
  EXPECT(nvfp4_quantize(F, NVFP4_IN_BF16, 64, 64, &c2, Ff, &out, NULL) == NVFP4_ERR_UNSUPPORTED);
  c2 = cfg;
  c2.emit_rowwise = 0;
  EXPECT(nvfp4_quantize(F, NVFP4_IN_BF16, 64, 64, &c2, Ff, &out, NULL) == NVFP4_ERR_UNSUPPORTED);
  nvfp4_outputs o2 = out;
  o2.codes_row = NULL;
  EXPECT(nvfp4_quantize(F, NVFP4_IN_BF16, 64, 64, &cfg, Ff, &o2, NULL) == NVFP4_ERR_NULL);
  o2 = out;
  o2.codes_row = ((uint8_t*)(U));
  EXPECT(nvfp4_quantize(F, NVFP4_IN_BF16, 64, 64, &cfg, Ff, &o2, NULL) == NVFP4_ERR_ALIGN);
  /* row offsets near the int64 limit: the element index would overflow */
  c2 = cfg;
  c2.sr = 1;
  c2.row_offset = INT64_MAX / 2;
  EXPECT(nvfp4_quantize(F, NVFP4_IN_BF16, 64, 64, &c2, Ff, &out, NULL) == NVFP4_ERR_SHAPE);
  c2.row_offset = -1;
  EXPECT(nvfp4_quantize(F, NVFP4_IN_BF16, 64, 64, &c2, Ff, &out, NULL) == NVFP4_ERR_SHAPE);

  /* dequantize */
  EXPECT(nvfp4_dequantize(F8, F8, Ff, 16, 24, NVFP4_BLOCK_1D, Ff, NULL) == NVFP4_ERR_SHAPE);
  EXPECT(nvfp4_dequantize(F8, F8, Ff, 8, 32, NVFP4_BLOCK_2D, Ff, NULL) == NVFP4_ERR_SHAPE);
  EXPECT(nvfp4_dequantize(F8, F8, Ff, 16, 32, (nvfp4_block)(3), Ff, NULL) == NVFP4_ERR_UNSUPPORTED);
  EXPECT(nvfp4_dequantize(NULL, F8, Ff, 16, 32, NVFP4_BLOCK_1D, Ff, NULL) == NVFP4_ERR_NULL);
  EXPECT(nvfp4_dequantize(((uint8_t*)(U)), F8, Ff, 16, 32, NVFP4_BLOCK_1D, Ff, NULL) == NVFP4_ERR_ALIGN);
  EXPECT(nvfp4_dequantize(F8, F8, Ff, 0, 32, NVFP4_BLOCK_1D, Ff, NULL) == NVFP4_OK);

  /* error statistics */
  EXPECT(nvfp4_error_stats(F, NVFP4_IN_BF16, 8, 64, &cfg, Ff, 0.25f, 26, ((double*)(F)), NULL) ==
         NVFP4_ERR_SHAPE);
  EXPECT(nvfp4_error_stats(F, NVFP4_IN_BF16, 64, 64, &cfg, Ff, 0.3f, 26, ((double*)(F)), NULL) ==
         NVFP4_ERR_UNSUPPORTED);
  EXPECT(nvfp4_error_stats(F, NVFP4_IN_BF16, 64, 64, &cfg, Ff, 0.25f, 65, ((double*)(F)), NULL) ==
         NVFP4_ERR_UNSUPPORTED);
  EXPECT(nvfp4_error_stats(F, NVFP4_IN_BF16, 64, 64, &cfg, Ff, 0.25f, 26, NULL, NULL) == NVFP4_ERR_NULL);

  /* MXFP4 */
  nvfp4_mx_config mc = {1, 0, 0, 0, 0};
  nvfp4_mx_outputs mo = {F8, F8, F8, F8};
  EXPECT(nvfp4_mxfp4_quantize(F, NVFP4_IN_BF16, 64, 48, &mc, &mo, NULL) == NVFP4_ERR_SHAPE);
  mc.emit_colwise = 1;
  EXPECT(nvfp4_mxfp4_quantize(F, NVFP4_IN_BF16, 48, 64, &mc, &mo, NULL) == NVFP4_ERR_SHAPE);
  EXPECT(nvfp4_mxfp4_quantize(F, NVFP4_IN_BF16, 0, 64, &mc, &mo, NULL) == NVFP4_OK);
  mc.emit_rowwise = mc.emit_colwise = 0;
  EXPECT(nvfp4_mxfp4_quantize(F, NVFP4_IN_BF16, 64, 64, &mc, &mo, NULL) == NVFP4_ERR_UNSUPPORTED);
  EXPECT(nvfp4_mxfp4_dequantize(F8, F8, 32, 48, Ff, NULL) == NVFP4_ERR_SHAPE);
  EXPECT(nvfp4_mxfp4_dequantize(F8, F8, 32, 32, ((float*)(U)), NULL) == NVFP4_ERR_ALIGN);

  /* GEMMs */
  EXPECT(nvfp4_gemm(F8, F8, Ff, NVFP4_BLOCK_1D, F8, F8, Ff, NVFP4_BLOCK_1D, 64, 64, 192, Ff, NULL) ==
         NVFP4_ERR_SHAPE);
  EXPECT(nvfp4_gemm(F8, F8, Ff, NVFP4_BLOCK_2D, F8, F8, Ff, NVFP4_BLOCK_1D, 8, 64, 128, Ff, NULL) ==
         NVFP4_ERR_SHAPE);
  EXPECT(nvfp4_gemm(NULL, F8, Ff, NVFP4_BLOCK_1D, F8, F8, Ff, NVFP4_BLOCK_1D, 64, 64, 128, Ff, NULL) ==
         NVFP4_ERR_NULL);
  EXPECT(nvfp4_gemm(F8, F8, Ff, NVFP4_BLOCK_1D, F8, F8, Ff, NVFP4_BLOCK_1D, 0, 64, 128, Ff, NULL) == NVFP4_OK);
  EXPECT(nvfp4_gemm(F8, F8, Ff, (nvfp4_block)(-1), F8, F8, Ff, NVFP4_BLOCK_1D, 64, 64, 128, Ff, NULL) ==
         NVFP4_ERR_UNSUPPORTED);
  EXPECT(nvfp4_gemm(F8, F8, Ff, NVFP4_BLOCK_1D, F8, F8, Ff, NVFP4_BLOCK_1D, 1ll << 40, 64, 128, Ff, NULL) ==
         NVFP4_ERR_SHAPE);
  EXPECT(nvfp4_mxfp4_gemm(F8, F8, F8, F8, 64, 64, 96, Ff, NULL) == NVFP4_ERR_SHAPE);
  EXPECT(nvfp4_mxfp4_gemm(F8, F8, ((uint8_t*)(U)), F8, 64, 64, 128, Ff, NULL) == NVFP4_ERR_ALIGN);

  if (failures) {
    fprintf(stderr, "%d expectation(s) failed\n", failures);
    return 1;
  }
  printf("abi driver: all rejections clean\n");
  return 0;
}
