/*
 * nvfp4.h -- C ABI of the MI355X (gfx950) NVFP4 block-quantization library
 * (libnvfp4.so).
 *
 * NVFP4 stores a tensor as 4-bit E2M1 codes (grid {0, 0.5, 1, 1.5, 2, 3, 4, 6},
 * sign bit 3), one E4M3 scale per 16-element block (or per 16x16 tile) and one
 * FP32 tensor scale.  Sources, cited by page title and section:
 *   [P1] "Pretraining Large Language Models with NVFP4" (explainer page):
 *        section 1 (16-element blocks with E4M3 scales), 2b (random Hadamard
 *        transform for gradients), 2c (2D block scaling keeps the row-wise and
 *        column-wise copies consistent), 2d (stochastic rounding).
 *   [P2] "Technical summary: Four Over Six (4/6)": "Problem statement" (E2M1
 *        grid; block max scaled to 6), "Core mechanism" (selected blocks scaled
 *        to 4), "Adaptive block scaling algorithm" (quantize with both scales,
 *        measure the error against the original values, keep the smaller under
 *        a max-error, MAE or MSE rule), "Implementation details" (tensor scale
 *        computed against an E4M3 limit of 256 instead of 448).
 *
 * Conventions for every entry point:
 *   - Tensors are row-major rows x cols (cols contiguous).  All data pointers
 *     are DEVICE pointers owned by the caller; the library allocates nothing
 *     and keeps no mutable global state (except the per-GPU scratch array of
 *     nvfp4_amax_noalloc, described there).
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Work is enqueued asynchronously on it; results are ready when the stream
 *     is synchronised.
 *   - Arguments are validated on the host before anything is launched: a
 *     non-OK status means nothing was enqueued.  NVFP4_ERR_HIP reports a launch
 *     failure (hipGetLastError).
 *   - Inputs must be finite.  Non-finite inputs give unspecified codes.
 *   - Arithmetic is IEEE binary32 with round-to-nearest-even per operation in
 *     a fixed order, so results are bit-reproducible run to run.
 */
#ifndef NVFP4_H
#define NVFP4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define NVFP4_ABI_VERSION 2

typedef enum {
  NVFP4_OK = 0,
  NVFP4_ERR_NULL = 1,        /* a required pointer is NULL */
  NVFP4_ERR_SHAPE = 2,       /* negative dims, or a dim not a multiple of 16 where blocks need it */
  NVFP4_ERR_ALIGN = 3,       /* a tensor pointer is not 16-byte aligned */
  NVFP4_ERR_DTYPE = 4,       /* unknown input dtype */
  NVFP4_ERR_UNSUPPORTED = 5, /* invalid option combination or value */
  NVFP4_ERR_WORKSPACE = 6,   /* workspace missing or too small */
  NVFP4_ERR_HIP = 7          /* a HIP launch failed */
} nvfp4_status;

typedef enum { NVFP4_IN_BF16 = 0, NVFP4_IN_F32 = 1 } nvfp4_dtype;

/* [P1] section 1 (1x16 blocks) and section 2c (16x16 tiles, one scale per tile). */
typedef enum { NVFP4_BLOCK_1D = 0, NVFP4_BLOCK_2D = 1 } nvfp4_block;

/* [P2] "Adaptive block scaling algorithm", step 3: the selection rules. */
typedef enum {
  NVFP4_RULE_NONE = 0,   /* standard NVFP4: every block's max is scaled to 6 */
  NVFP4_RULE_MSE = 1,    /* keep the candidate with the smaller sum of squared errors */
  NVFP4_RULE_MAE = 2,    /* ... smaller sum of absolute errors */
  NVFP4_RULE_MAXERR = 3  /* ... smaller maximum absolute error */
} nvfp4_rule;

typedef struct {
  int32_t block;          /* nvfp4_block */
  int32_t emit_rowwise;   /* write the row-wise copy (blocks along cols) */
  int32_t emit_colwise;   /* write the column-wise copy, laid out as the transpose */
  int32_t rht;            /* 16-point random Hadamard transform on each 1x16 row block
                             before quantization ([P1] 2b); row-wise 1D only */
  uint16_t rht_sign_mask; /* bit i set: element i of each block is negated before the transform */
  int32_t sr;             /* 1: stochastic rounding ([P1] 2d); 0: round to nearest even */
  uint64_t sr_seed;       /* Philox-4x32-10 key for stochastic rounding */
  int64_t row_offset;     /* global row of row 0: element (r, c) has index (row_offset + r) * cols + c,
                             which keys its random word; 0 for an unsharded tensor */
  int32_t rule;           /* nvfp4_rule: the Four Over Six choice ([P2]) */
  float scale_cap;        /* E4M3 limit for the tensor scale: 448 (standard) or 256 ([P2]
                             "Implementation details": leaves room for the 1.5x larger
                             factor of a block scaled to 4) */
} nvfp4_config;

/* Device output buffers for nvfp4_quantize.  A copy not requested may be NULL.
 *   codes_row   [rows][cols/2]      two codes per byte: element 2k in bits 0-3, 2k+1 in bits 4-7
 *   scales_row  [rows][cols/16]     E4M3 block scales (2D: [rows/16][cols/16], one per tile)
 *   codes_col   [cols][rows/2]      the column-wise copy: codes of x^T in the same packing
 *   scales_col  [cols][rows/16]     (2D: [cols/16][rows/16], the transposed tile grid)
 *   tensor_scale                    one float: S_t = amax / (6 * scale_cap)
 * codes_* must be 16-byte aligned; scales_* and tensor_scale need natural alignment only. */
typedef struct {
  uint8_t* codes_row;
  uint8_t* scales_row;
  uint8_t* codes_col;
  uint8_t* scales_col;
  float* tensor_scale;
} nvfp4_outputs;

/* Bytes of device workspace nvfp4_amax needs for this shape (a few KB). */
size_t nvfp4_amax_workspace_bytes(int64_t rows, int64_t cols);

/* Per-tensor amax: *amax_dev = max |y| over the tensor, y = x, or y = the
 * Hadamard-transformed row blocks when cfg->rht is set (the tensor scale must
 * cover the values actually quantized).  [P2] "Implementation details" (the
 * FP32 tensor scale is derived from it).
 *   x          device, 16-byte aligned, rows x cols of `dtype`
 *   cfg        host pointer; only rht and rht_sign_mask are read (NULL = no transform)
 *   amax_dev   device, one float, written
 *   workspace  device, at least nvfp4_amax_workspace_bytes(rows, cols) bytes, any contents
 * An empty tensor (rows or cols == 0) gives amax 0.  With rht, cols % 16 == 0. */
nvfp4_status nvfp4_amax(const void* x, nvfp4_dtype dtype, int64_t rows, int64_t cols, const nvfp4_config* cfg,
                        float* amax_dev, void* workspace, size_t workspace_bytes, void* stream);

/* nvfp4_amax without a workspace, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  Same arguments, kernels and result as nvfp4_amax; the partial
 * maxima go to a 4 KB array the library keeps in each GPU's memory until the
 * process ends (nothing is allocated by the call; any tensor size is accepted,
 * since the number of partials is capped).  Every call on one GPU shares that
 * array: calls that overlap on one GPU (different streams or threads) race, and
 * must be ordered by the caller.  NVFP4_ERR_HIP if the array's address cannot be
 * obtained on the stream's device; NVFP4_ERR_UNSUPPORTED for device ordinals
 * of 64 and above. */
nvfp4_status nvfp4_amax_noalloc(const void* x, nvfp4_dtype dtype, int64_t rows, int64_t cols,
                                const nvfp4_config* cfg, float* amax_dev, void* stream);

/* Quantize x into NVFP4 with one fused pass over the input.
 * Per block (1x16 row block, 16x1 column block, or 16x16 tile):
 *   S_t = fl(amax / fl(6 * scale_cap))
 *   candidate T in {6} (plus {4} when rule != NONE, [P2] "Adaptive block scaling" step 1):
 *     r = fl(m_b / fl(T * S_t)) with m_b = max |y| over the block (0 if m_b or the divisor is 0)
 *     sb = E4M3 round-to-nearest-even of r, saturating at 448
 *     d = fl(dec(sb) * S_t);  e = fl(1 / d) (0 when d = 0 or 1/d overflows)
 *     code_i = E2M1 rounding of fl(y_i * e): nearest, ties to even (sr = 0), or
 *              stochastic with the element's Philox word (sr = 1)
 *   with a rule, the error of each candidate against y ([P2] step 2) is
 *     eps_i = fl(y_i - fl(value(code_i) * d)); MSE / MAE: pairwise sum (index order) of
 *     eps_i^2 / |eps_i|; MAXERR: max |eps_i|.  T = 4 is kept iff its error is strictly smaller.
 * Stochastic rounding: the element with index idx = (row_offset + r) * cols + c uses word
 *   (idx mod 4) of Philox-4x32-10 at key (sr_seed low, high), counter (q low, q high, 0, 0),
 *   q = idx / 4; it rounds up iff (word >> 10) + floor(f * 2^22) >= 2^22, f the fractional
 *   distance to the next grid point.  Both copies use the element's word; with a 4/6 rule the
 *   scale-to-4 candidate rounds with the word shifted left by one (its bits 30..9).
 * Shapes: cols % 16 == 0; rows % 16 == 0 and cols <= 2^24 when a column copy or 2D tiles are
 * requested; rows * cols <= 2^60; row_offset >= 0 and (row_offset + rows) * cols <= 2^62
 * (NVFP4_ERR_SHAPE otherwise).
 * Unsupported (NVFP4_ERR_UNSUPPORTED): rht with 2D or with a column copy; scale_cap other than
 * 448 or 256; no copy requested; an unknown rule or block kind.
 *   x          device, 16-byte aligned
 *   cfg        host pointer
 *   amax_dev   device, one float (e.g. from nvfp4_amax, or a caller-provided amax)
 *   out        host pointer to device buffers (see nvfp4_outputs) */
nvfp4_status nvfp4_quantize(const void* x, nvfp4_dtype dtype, int64_t rows, int64_t cols, const nvfp4_config* cfg,
                            const float* amax_dev, const nvfp4_outputs* out, void* stream);

/* Dequantize an NVFP4 copy back to binary32.  [P1] section 1: each 16-element
 * block (or 16x16 tile, section 2c) carries one E4M3 scale; [P2]
 * "Implementation details": one FP32 tensor scale S_t multiplies every block
 * scale.  So an element decodes to its E2M1 value times dec(sb) * S_t:
 *   out[r][c] = fl(value(code) * fl(dec(sb) * S_t)), the same value the 4/6 error used.
 *   codes        device [rows][cols/2], 16-byte aligned
 *   scales       device [rows][cols/16] (block 1D) or [rows/16][cols/16] (block 2D)
 *   tensor_scale device, one float (S_t as written by nvfp4_quantize)
 *   out          device float [rows][cols], 16-byte aligned
 * A column-wise copy is dequantized by passing its own dims (rows = original cols). */
nvfp4_status nvfp4_dequantize(const uint8_t* codes, const uint8_t* scales, const float* tensor_scale, int64_t rows,
                              int64_t cols, nvfp4_block block, float* out, void* stream);

/* Sign mask for the Hadamard transform derived from a seed ([P1] section 2b:
 * the transform is randomized by a seeded sign vector; one sign per element
 * of the 16-point block): the low 16 bits of word 0 of Philox-4x32-10 at key
 * (seed low, seed high), counter (0, 0, 0, 1) (stochastic rounding only uses
 * counters whose last word is 0). */
uint16_t nvfp4_rht_signs_from_seed(uint64_t seed);

/* ---- error analysis ----------------------------------------------------------
 * [P2] "Problem statement": the error of values near the block max (around the
 * scaled value 5) dominates, and the quantization of the scale factor itself
 * matters little.  This call measures both on a tensor.  It quantizes x with
 * round-to-nearest exactly as nvfp4_quantize does (cfg->block, rht, rule and
 * scale_cap; 1x16 row blocks or 16x16 tiles; sr must be 0 and the emit flags
 * are ignored) and bins every element by its scaled value |z|, z = fl(y * e), in
 * bins [k * bin_width, (k + 1) * bin_width) (the last bin takes everything
 * above).  stats_dev receives three rows of nbins doubles:
 *   [0][k]  number of elements in bin k (exact)
 *   [1][k]  sum of eps^2, eps = fl(y - fl(v * d)) (the dequantized error)
 *   [2][k]  sum of eps*^2 for a reference with an unquantized scale: the block max
 *           maps exactly onto the chosen T, v* = nearest-even E2M1 of T|y| / m_b,
 *           eps* = fl64(y - fl64(v* * m_b / T)) with the sign of y
 * Sums are accumulated in binary64 in an unspecified order: each sum of n terms
 * is within a relative n * 2^-53 of the exact one.  The call overwrites all
 * 3 * nbins values.  rows % 16 == 0, cols % 16 == 0; bin_width a power of two;
 * 1 <= nbins <= 64 (NVFP4_ERR_UNSUPPORTED otherwise, also for sr or rht with 2D).
 *   x          device, 16-byte aligned;  cfg: host pointer
 *   amax_dev   device, one float (the tensor amax, e.g. from nvfp4_amax)
 *   stats_dev  device, 3 * nbins doubles */
nvfp4_status nvfp4_error_stats(const void* x, nvfp4_dtype dtype, int64_t rows, int64_t cols, const nvfp4_config* cfg,
                               const float* amax_dev, float bin_width, int32_t nbins, double* stats_dev,
                               void* stream);

/* ---- MXFP4 -----------------------------------------------------------------
 * The format [P1] section 1 contrasts with NVFP4: 32-element blocks, each with
 * a power-of-two scale stored as E8M0 (2^(code - 127); code 255 is NaN), and no
 * tensor scale.  The pages do not give its scale rule; the library follows the
 * OCP Microscaling v1.0 one: for block max m, the shared exponent is
 * floor(log2 m) - 2 (2 being the largest E2M1 exponent), clamped to >= -127
 * (m = 0 and m < 2^-125 give code 0).  Elements: E2M1 of fl(y * 2^-e),
 * nearest-even or stochastic with the element's Philox word exactly as in
 * nvfp4_quantize (the same key, counter and decision rule).  Four Over Six
 * does not apply ([P2]: the power-of-two scale has no room for it). */
typedef struct {
  int32_t emit_rowwise;  /* 1x32 row blocks */
  int32_t emit_colwise;  /* 32x1 column blocks, laid out as the transpose */
  int32_t sr;            /* 1: stochastic rounding; 0: round to nearest even */
  uint64_t sr_seed;
  int64_t row_offset;    /* as in nvfp4_config (the same limits) */
} nvfp4_mx_config;

/* Device outputs of nvfp4_mxfp4_quantize (a copy not requested may be NULL):
 *   codes_row  [rows][cols/2]   packed like nvfp4_outputs
 *   scales_row [rows][cols/32]  E8M0 codes
 *   codes_col  [cols][rows/2]
 *   scales_col [cols][rows/32]
 * codes_* must be 16-byte aligned. */
typedef struct {
  uint8_t* codes_row;
  uint8_t* scales_row;
  uint8_t* codes_col;
  uint8_t* scales_col;
} nvfp4_mx_outputs;

/* One pass over x, no amax needed.  Shapes: cols % 32 == 0; rows % 32 == 0 and
 * cols <= 2^24 with a column copy.  NVFP4_ERR_UNSUPPORTED if no copy is requested.
 *   x    device, 16-byte aligned;  cfg, out: host pointers */
nvfp4_status nvfp4_mxfp4_quantize(const void* x, nvfp4_dtype dtype, int64_t rows, int64_t cols,
                                  const nvfp4_mx_config* cfg, const nvfp4_mx_outputs* out, void* stream);

/* out[r][c] = value(code) * 2^(sc - 127) (exact; NaN where sc == 255).
 *   codes device [rows][cols/2], 16-byte aligned; scales device [rows][cols/32];
 *   out device float [rows][cols], 16-byte aligned; cols % 32 == 0.  A column copy
 *   is dequantized with its own dims (rows = original cols). */
nvfp4_status nvfp4_mxfp4_dequantize(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t cols,
                                    float* out, void* stream);

/* ---- the consumer: FP4 GEMM ---------------------------------------------------
 * [P4] (the news page "NVFP4 revolutionizes AI training", title translated)
 * gives fast FP4 matrix products as the reason for the format.  Both calls
 * compute C = A B^T from quantized row copies with K contiguous ("NT"):
 *   A codes [M][K/2], B codes [N][K/2] (as written by the quantize calls),
 *   C float [M][N] row-major, overwritten.
 * The result is the value the operands encode, summed with fp32 accumulation
 * on the matrix cores: each instruction adds its exact products to the running
 * sum with at most one unit of 2^-24 of (|running sum| + sum |products|) of
 * error (measured), so |C - exact| <= 2 (K / k_i) 2^-24 sum_k |A B|, with k_i =
 * 64 values per instruction for MXFP4 and 16 for NVFP4 (plus one unit of |C|
 * for NVFP4's tensor-scale multiply).  Deterministic run to run.
 * Pointers: codes 16-byte aligned, scales and C 4-byte aligned.  M, N, K <= 2^31.
 *
 * NVFP4: scales [M][K/16] / [N][K/16] (NVFP4_BLOCK_1D) or [M/16][K/16] /
 *   [N/16][K/16] (NVFP4_BLOCK_2D, e.g. the column copy of a 16x16-tiled weight);
 *   a_tensor_scale, b_tensor_scale: device floats.  K % 128 == 0; M % 16 == 0 with
 *   2D A, N % 16 == 0 with 2D B.  C = S_tA S_tB sum_k (v dec(sb))_A (v dec(sb))_B. */
nvfp4_status nvfp4_gemm(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_tensor_scale,
                        nvfp4_block a_block, const uint8_t* b_codes, const uint8_t* b_scales,
                        const float* b_tensor_scale, nvfp4_block b_block, int64_t M, int64_t N, int64_t K, float* c,
                        void* stream);

/* MXFP4: scales [M][K/32] and [N][K/32] (E8M0); K % 128 == 0.
 * C = sum_k v_A 2^(sA - 127) v_B 2^(sB - 127). */
nvfp4_status nvfp4_mxfp4_gemm(const uint8_t* a_codes, const uint8_t* a_scales, const uint8_t* b_codes,
                              const uint8_t* b_scales, int64_t M, int64_t N, int64_t K, float* c, void* stream);

const char* nvfp4_status_string(nvfp4_status s);
int nvfp4_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif
