/* Drives every oracle entry point over small tensors with ragged shapes and
 * every option, for a run under AddressSanitizer and UndefinedBehaviorSanitizer
 * on the CPU.  Inputs come from a fixed linear congruential sequence (no
 * quantization arithmetic here); the run passes when every call returns its
 * expected status and the sanitizers report nothing. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "nvfp4_oracle.h"

static uint64_t lcg = 88172645463325252ull;
static double uni(void) {
  lcg = lcg * 6364136223846793005ull + 1442695040888963407ull;
  return (double)(lcg >> 11) * 0x1p-53;
}

static void fill(float* x, int64_t n, double scale) {
  for (int64_t i = 0; i < n; ++i) {
    double v = (uni() - 0.5) * 2.0 * scale;
    if (uni() < 0.02) v *= 50.0;
    if (uni() < 0.01) v = 0.0;
    x[i] = (float)v;
  }
}

static void to_bf16(const float* x, uint16_t* h, int64_t n) {
  for (int64_t i = 0; i < n; ++i) {
    uint32_t b;
    memcpy(&b, &x[i], 4);
    h[i] = (uint16_t)(b >> 16);
  }
}

static int failures = 0;
#define EXPECT(cond)                                          \
  do {                                                        \
    if (!(cond)) {                                            \
      fprintf(stderr, "failed: %s (line %d)\n", #cond, __LINE__); \
      ++failures;                                             \
    }                                                         \
  } while (0)

static void run_quantize(int64_t M, int64_t N, int dtype, int block_2d, int row, int col, int rht, int sr, int rule,
                         float cap, int64_t row_offset, int threads) {
  float* xf = (float*)malloc(sizeof(float) * (size_t)(M * N) + 1);
  uint16_t* xh = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)(M * N) + 1);
  fill(xf, M * N, 3.0);
  to_bf16(xf, xh, M * N);
  const void* x = dtype == ORC_IN_F32 ? (const void*)xf : (const void*)xh;
  orc_config cfg = {block_2d, row, col, rht, 0xB3E1u, sr, 12345u, row_offset, rule, cap};
  float A = orc_amax(x, dtype, M, N, rht, cfg.rht_mask);
  const int64_t sb_row = block_2d ? (M / 16) * (N / 16) : M * (N / 16);
  const int64_t sb_col = block_2d ? (N / 16) * (M / 16) : N * (M / 16);
  uint8_t* cr = row ? (uint8_t*)calloc((size_t)(M * N / 2) + 1, 1) : NULL;
  uint8_t* sr_ = row ? (uint8_t*)calloc((size_t)sb_row + 1, 1) : NULL;
  uint8_t* pr = row ? (uint8_t*)calloc((size_t)sb_row + 1, 1) : NULL;
  uint8_t* cc = col ? (uint8_t*)calloc((size_t)(M * N / 2) + 1, 1) : NULL;
  uint8_t* sc = col ? (uint8_t*)calloc((size_t)sb_col + 1, 1) : NULL;
  uint8_t* pc = col ? (uint8_t*)calloc((size_t)sb_col + 1, 1) : NULL;
  float ts = 0.0f;
  EXPECT(orc_quantize(x, dtype, M, N, &cfg, A, cr, sr_, cc, sc, &ts, pr, pc, threads) == 0);
  if (row) {
    float* dq = (float*)malloc(sizeof(float) * (size_t)(M * N) + 1);
    orc_dequantize(cr, sr_, ts, M, N, block_2d, dq);
    for (int64_t i = 0; i < M * N; ++i) EXPECT(isfinite(dq[i]));
    free(dq);
  }
  if (!sr && !(rht && block_2d) && M % 16 == 0) {
    double stats[3 * 26];
    EXPECT(orc_error_stats(x, dtype, M, N, &cfg, A, 0.25f, 26, stats) == 0);
  }
  free(xf), free(xh), free(cr), free(sr_), free(pr), free(cc), free(sc), free(pc);
}

int main(void) {
  /* format functions over special values */
  const float specials[] = {0.0f, -0.0f, 0.25f, 0.75f, 5.0f, 6.0f, 7.9f, 1e30f, -1e-40f, INFINITY, 448.0f, 465.0f};
  for (size_t i = 0; i < sizeof(specials) / sizeof(specials[0]); ++i) {
    (void)orc_e2m1_rne(specials[i]);
    (void)orc_e2m1_sr(specials[i], 0xFFFFFFFFu);
    if (specials[i] >= 0.0f) (void)orc_e4m3_rne_sat(specials[i]);
    (void)orc_mx_scale_code(fabsf(specials[i]));
  }
  for (int c = 0; c < 256; ++c) {
    (void)orc_e4m3_value((uint8_t)c);
    (void)orc_e8m0_value((uint8_t)c);
    if (c < 16) (void)orc_e2m1_value((uint8_t)c);
  }
  /* every option on ragged and multi-tile shapes, both dtypes, 1 and 3 threads */
  const int64_t shapes[][2] = {{16, 16}, {48, 80}, {33, 48}, {64, 208}, {0, 32}};
  for (size_t s = 0; s < sizeof(shapes) / sizeof(shapes[0]); ++s) {
    const int64_t M = shapes[s][0], N = shapes[s][1];
    for (int dtype = 0; dtype < 2; ++dtype)
      for (int rule = 0; rule < 4; ++rule)
        for (int sr = 0; sr < 2; ++sr) {
          const float cap = rule ? 256.0f : 448.0f;
          run_quantize(M, N, dtype, 0, 1, 0, 0, sr, rule, cap, 0, 1);
          run_quantize(M, N, dtype, 0, 1, 0, 1, sr, rule, cap, 7, 3);
          if (M % 16 == 0) {
            run_quantize(M, N, dtype, 0, 1, 1, 0, sr, rule, cap, (1ll << 30) + 5, 3);
            run_quantize(M, N, dtype, 1, 1, 1, 0, sr, rule, cap, 0, 2);
          }
        }
  }
  /* rejected configurations return an error without touching the buffers */
  {
    float x[16 * 24];
    fill(x, 16 * 24, 1.0);
    orc_config bad = {0, 1, 0, 0, 0, 0, 0, 0, 0, 448.0f};
    EXPECT(orc_quantize(x, ORC_IN_F32, 16, 24, &bad, 1.0f, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 1) != 0);
    bad.cap = 300.0f;
    EXPECT(orc_quantize(x, ORC_IN_F32, 16, 16, &bad, 1.0f, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 1) != 0);
  }
  /* MXFP4 and the GEMM consumer */
  {
    const int64_t M = 64, N = 96;
    float* x = (float*)malloc(sizeof(float) * M * N);
    fill(x, M * N, 2.0);
    uint8_t *cr = calloc(M * N / 2, 1), *sr = calloc(M * N / 32, 1), *cc = calloc(M * N / 2, 1),
            *sc = calloc(M * N / 32, 1);
    EXPECT(orc_mxfp4_quantize(x, ORC_IN_F32, M, N, 1, 1, 1, 9, 3, cr, sr, cc, sc) == 0);
    float* dq = malloc(sizeof(float) * M * N);
    orc_mxfp4_dequantize(cr, sr, M, N, dq);
    const int64_t K = 128, GM = 32, GN = 48;
    uint8_t *ac = calloc(GM * K / 2, 1), *as = calloc(GM * K / 16, 1), *bc = calloc(GN * K / 2, 1),
            *bs = calloc(GN * K / 16, 1);
    for (int64_t i = 0; i < GM * K / 2; ++i) ac[i] = (uint8_t)(uni() * 256);
    for (int64_t i = 0; i < GN * K / 2; ++i) bc[i] = (uint8_t)(uni() * 256);
    for (int64_t i = 0; i < GM * K / 16; ++i) as[i] = (uint8_t)(uni() * 126);
    for (int64_t i = 0; i < GN * K / 16; ++i) bs[i] = (uint8_t)(uni() * 126);
    float* c = malloc(sizeof(float) * GM * GN);
    double* cabs = malloc(sizeof(double) * GM * GN);
    EXPECT(orc_gemm_fp4(0, ac, as, 0.5f, 0, bc, bs, 2.0f, 0, GM, GN, K, c, cabs) == 0);
    EXPECT(orc_gemm_fp4(1, ac, as, 1.0f, 0, bc, bs, 1.0f, 0, GM, GN, K, c, cabs) == 0);
    EXPECT(orc_gemm_fp4(0, ac, as, 1.0f, 1, bc, bs, 1.0f, 1, GM, GN, K, c, NULL) == 0);
    free(x), free(cr), free(sr), free(cc), free(sc), free(dq), free(ac), free(as), free(bc), free(bs), free(c),
        free(cabs);
  }
  /* generators */
  {
    uint32_t ctr[4] = {1, 2, 3, 4}, key[2] = {5, 6}, out[4];
    orc_philox4x32_10(ctr, key, out);
    (void)orc_sr_word(0xFFFFFFFFFFFFFFFFull, 0xFFFFFFFFFFFFFFFFull);
    (void)orc_rht_mask_from_seed(1234);
  }
  if (failures) {
    fprintf(stderr, "%d expectation(s) failed\n", failures);
    return 1;
  }
  printf("oracle driver: all calls clean\n");
  return 0;
}
