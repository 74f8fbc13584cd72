/*
 * nvfp4_oracle.h -- plain CPU reference for NVFP4 block quantization.
 *
 * TEST INFRASTRUCTURE ONLY.  This oracle is the correctness reference that the
 * GPU path is compared against, element by element.  Only the test suite, the
 * package's smoke check and the benchmark's CPU-baseline leg may load it; the
 * product path never calls it and shares no code, header, table or helper with
 * it.
 *
 * Sources (web pages, cited by title and section):
 *   [P1] "Pretraining Large Language Models with NVFP4" (explainer page):
 *        section 1 (16-element blocks, E4M3 block scales), section 2b (random
 *        Hadamard transform), section 2c (2D block scaling), section 2d
 *        (stochastic rounding).
 *   [P2] "Technical summary: Four Over Six (4/6)": "Problem statement" (the E2M1
 *        grid and its step sizes, block max mapped to 6), "Core mechanism"
 *        (scaling selected blocks to 4), "Adaptive block scaling algorithm"
 *        (dual quantization, error against the original values, min max-error /
 *        MAE / MSE rules), "Implementation details" (tensor scale computed
 *        against an E4M3 limit of 256 instead of 448).
 *   [P1] section 1 also names MXFP4 as the contrast: 32-element blocks with a
 *        power-of-two (E8M0) scale.  The pages do not give its scale rule; the
 *        oracle takes the OCP Microscaling v1.0 one (shared exponent =
 *        floor(log2 of the block max) minus the largest E2M1 exponent, 2).
 *
 * Arithmetic: IEEE binary32, one rounding (to nearest even) per operation, in
 * the fixed order written in nvfp4_oracle.c.  Built with -ffp-contract=off and
 * without fast-math; denormals are kept.  Where a step has a plain
 * mathematical definition (nearest grid point, nearest E4M3 value) it is
 * evaluated exactly in binary64.
 *
 * Parity status of each function (what pins it is in the test suite):
 *   orc_e2m1_rne, orc_e2m1_value, orc_e4m3_*, orc_rht16, orc_amax,
 *   orc_quantize (RNE), orc_dequantize  -- pinned (page values, worked
 *       examples, brute force, library routines, closed forms).
 *   orc_philox4x32_10 -- pinned against an independent library implementation
 *       of the published Philox-4x32-10 generator.
 *   orc_e2m1_sr -- pinned statistically (unbiasedness) and by its special
 *       cases; the exact random-word-to-decision mapping is a reading, not a
 *       page fact.
 *   orc_gemm_fp4 -- pinned by numpy float64 matrix products of operands
 *       decoded through the pinned format functions, and closed forms.
 *   orc_error_stats -- pinned by the total squared error of orc_quantize +
 *       orc_dequantize, brute-force exact-scale rounding with rationals, and
 *       the concentration of error near the scaled value 5 that [P2]
 *       "Problem statement" reports.
 *   orc_mx_scale_code, orc_mxfp4_* -- pinned by brute force (nearest of the
 *       scaled grid), the defining range of the scaled block max, the
 *       row/column transpose identity and the outlier behaviour [P1] section 1
 *       describes; the scale rule itself is a reading (see above).
 *   op-order choices (block-scale division order, reciprocal-then-multiply,
 *       pairwise error sum) -- parity unpinned by the pages.
 */
#ifndef NVFP4_ORACLE_H
#define NVFP4_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORC_IN_BF16 = 0, ORC_IN_F32 = 1 };
enum { ORC_RULE_NONE = 0, ORC_RULE_MSE = 1, ORC_RULE_MAE = 2, ORC_RULE_MAXERR = 3 };

typedef struct {
  int32_t block_2d;   /* 0: 1x16 blocks; 1: 16x16 tiles with one scale each */
  int32_t emit_row;   /* write the row-wise copy */
  int32_t emit_col;   /* write the column-wise (transposed) copy */
  int32_t rht;        /* apply the 16-point random Hadamard transform (row-wise 1D only) */
  uint32_t rht_mask;  /* bit i set: negate element i of each 16-block before the transform */
  int32_t sr;         /* stochastic rounding instead of round-to-nearest-even */
  uint64_t sr_seed;   /* Philox key for stochastic rounding */
  int64_t row_offset; /* global row index of row 0 (element index = (row_offset+r)*cols + c) */
  int32_t rule;       /* ORC_RULE_*: 4/6 selection rule, NONE = always scale to 6 */
  float cap;          /* E4M3 limit used for the tensor scale: 448 or 256 */
} orc_config;

/* ---- number formats ---------------------------------------------------- */
float   orc_bf16_to_f32(uint16_t h);
uint8_t orc_e2m1_rne(float z);                 /* 4-bit code: sign<<3 | grid index */
uint8_t orc_e2m1_sr(float z, uint32_t rword);  /* stochastic rounding with one random word */
float   orc_e2m1_value(uint8_t code);
uint8_t orc_e4m3_rne_sat(float r);             /* r >= 0; RNE, saturating at 448 (0x7E) */
float   orc_e4m3_value(uint8_t code);

/* ---- randomness -------------------------------------------------------- */
void     orc_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]);
uint32_t orc_sr_word(uint64_t seed, uint64_t idx);
uint32_t orc_rht_mask_from_seed(uint64_t seed);

/* ---- transform --------------------------------------------------------- */
void orc_rht16(const float* x, uint32_t mask, float* y);

/* ---- block level (exposed for the pins) -------------------------------- */
/* Quantize one block of n (16 or 256) values y with tensor scale s_t.
 * rwords: one random word per element (used only when sr != 0; may be NULL otherwise);
 * the scale-to-6 candidate rounds with the word itself, the scale-to-4 candidate
 * with the word shifted left by one (bits 30..9 become the 22-bit threshold).
 * Outputs: codes[n], *scale (E4M3 code), *chose4 (1 if the scale-to-4 candidate won),
 * err[0] = error of the scale-to-6 candidate, err[1] = scale-to-4 (0 when rule == NONE). */
void orc_quantize_block(const float* y, int n, float s_t, int rule, int sr, const uint32_t* rwords,
                        uint8_t* codes, uint8_t* scale, uint8_t* chose4, float* err);

/* ---- tensor level ------------------------------------------------------ */
float orc_amax(const void* x, int dtype, int64_t rows, int64_t cols, int rht, uint32_t mask);
float orc_tensor_scale(float amax, float cap);

/* Returns 0 on success, nonzero on a shape/config violation.
 * Layouts: codes_row [rows][cols/2]; scales_row [rows][cols/16] (2D: [rows/16][cols/16]);
 * codes_col [cols][rows/2]; scales_col [cols][rows/16] (2D: [cols/16][rows/16]).
 * Nibbles: element 2k in bits 0-3 of byte k, element 2k+1 in bits 4-7.
 * pick_row / pick_col (optional, may be NULL): one byte per block, 1 if scale-to-4 won.
 * nthreads: row bands processed by that many threads (bands are whole 16-row groups). */
int orc_quantize(const void* x, int dtype, int64_t rows, int64_t cols, const orc_config* cfg, float amax,
                 uint8_t* codes_row, uint8_t* scales_row, uint8_t* codes_col, uint8_t* scales_col,
                 float* tensor_scale, uint8_t* pick_row, uint8_t* pick_col, int nthreads);

/* codes [rows][cols/2], scales as above for the given block kind; out [rows][cols] */
void orc_dequantize(const uint8_t* codes, const uint8_t* scales, float tensor_scale, int64_t rows, int64_t cols,
                    int block_2d, float* out);

/* ---- error analysis ([P2] "Problem statement": the error of values near the
 * block max, around the scaled value 5, dominates; the scale factor's own
 * quantization matters little) ------------------------------------------------
 * Round-to-nearest NVFP4 as orc_quantize computes it (1x16 row blocks, with the
 * transform if cfg->rht, or 16x16 tiles; cfg->rule chooses 4/6), plus a
 * reference with an exact scale (the block max maps exactly to the chosen T).
 * Elements are binned by their scaled value |z| in bins of width bin_width (a
 * power of two; the last bin takes everything above).  stats[3][nbins]
 * (binary64): element count, sum of eps^2, sum of eps*^2 (exact-scale error).
 * rows % 16 == 0, cols % 16 == 0, 1 <= nbins <= 64, no stochastic rounding. */
int orc_error_stats(const void* x, int dtype, int64_t rows, int64_t cols, const orc_config* cfg, float amax,
                    float bin_width, int nbins, double* stats);

/* ---- the consumer: GEMM on FP4 operands ([P4], the news page "NVFP4
 * revolutionizes AI training" (title translated): the format exists for fast
 * FP4 matrix products) ----------------------------------------------------
 * C[m][n] = sum_k A[m][k] * B[n][k] ("NT": both operands stored with K
 * contiguous, as quantized row copies), where an operand element is the value
 * its encoding stands for: NVFP4 v * dec(sb) * S_t (scales [rows][K/16], or
 * [rows/16][K/16] for 16x16 tiles), MXFP4 v * 2^(sc - 127) (scales [rows][K/32]).
 * Products are exact in binary64 and summed in k order in binary64; the tensor
 * scales multiply the sum; one rounding to binary32 at the end.  c_abs (may be
 * NULL) receives sum_k |A B| (with the tensor scales), for error bounds.
 * mx = 1: MXFP4 operands (a_ts, b_ts, a_2d, b_2d ignored). */
int orc_gemm_fp4(int mx, const uint8_t* a_codes, const uint8_t* a_scales, float a_ts, int a_2d, const uint8_t* b_codes,
                 const uint8_t* b_scales, float b_ts, int b_2d, int64_t M, int64_t N, int64_t K, float* c,
                 double* c_abs);

/* ---- MXFP4 (the contrast format of [P1] section 1) ----------------------
 * OCP Microscaling (MX) FP4: 32-element row blocks, each with a power-of-two
 * scale X = 2^e stored as E8M0 (biased exponent e + 127), no tensor scale.
 * e = floor(log2(max |y|)) - 2 (2 = the largest exponent of E2M1), clamped to
 * [-127, 127]; an all-zero block gets e = -127.  Elements: E2M1 rounding of
 * y / X (nearest-even or stochastic as above), saturating at 6.
 * Row copy: codes [rows][cols/2] (same packing), scales [rows][cols/32],
 * cols % 32 == 0.  Column copy (blocks of 32 rows, stored transposed): codes
 * [cols][rows/2], scales [cols][rows/32], rows % 32 == 0.  Stochastic rounding
 * uses the element's word from orc_sr_word, as in NVFP4. */
float orc_e8m0_value(uint8_t code);
uint8_t orc_mx_scale_code(float block_max);
int orc_mxfp4_quantize(const void* x, int dtype, int64_t rows, int64_t cols, int emit_row, int emit_col, int sr,
                       uint64_t sr_seed, int64_t row_offset, uint8_t* codes_row, uint8_t* scales_row,
                       uint8_t* codes_col, uint8_t* scales_col);
void orc_mxfp4_dequantize(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t cols, float* out);

/* ---- batch forms of the scalar functions above (same semantics) -------- */
void orc_e2m1_rne_n(const float* z, int64_t n, uint8_t* out);
void orc_e2m1_sr_n(const float* z, const uint32_t* w, int64_t n, uint8_t* out);
void orc_e4m3_rne_sat_n(const float* r, int64_t n, uint8_t* out);
void orc_sr_words_n(uint64_t seed, const uint64_t* idx, int64_t n, uint32_t* out);
void orc_philox_n(const uint32_t* ctr, const uint32_t* key, int64_t n, uint32_t* out);

#ifdef __cplusplus
}
#endif
#endif
