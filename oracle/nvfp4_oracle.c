/*
 * nvfp4_oracle.c -- plain CPU reference for NVFP4 block quantization.
 * TEST INFRASTRUCTURE ONLY (see nvfp4_oracle.h): never called by the product path.
 *
 * Build: gcc -std=c11 -O2 -ffp-contract=off -fno-fast-math -fPIC -shared -pthread
 *
 * Every floating-point step below is written as one binary32 operation in the
 * order stated; fl(.) in the comments means "rounded to binary32, to nearest
 * even".  Steps with a plain mathematical definition (nearest point of a finite
 * grid) are evaluated exactly in binary64.
 */
#include "nvfp4_oracle.h"

#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* Number formats                                                            */
/* ------------------------------------------------------------------------ */

/* bf16 is the upper half of a binary32 pattern: widening is exact. */
float orc_bf16_to_f32(uint16_t h) {
  uint32_t b = (uint32_t)h << 16;
  float f;
  memcpy(&f, &b, 4);
  return f;
}

/* The E2M1 magnitudes.  [P2] "Problem statement": steps of 0.5 on [0,2],
 * 1 on [2,4] and 2 on [4,6]; the largest value is 6. */
static const double kE2M1[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

static int sign_bit(float z) {
  uint32_t b;
  memcpy(&b, &z, 4);
  return (int)(b >> 31);
}

/* Round to nearest E2M1 magnitude; on an exact tie take the even grid index.
 * Anything at or beyond 6 is nearest to 6 (taken directly: for huge |z| the
 * binary64 differences below would no longer be exact).
 * The sign bit of z is kept, so -0 and small negatives give code 0x8. */
uint8_t orc_e2m1_rne(float z) {
  double a = fabs((double)z);
  if (a >= 6.0) return (uint8_t)((sign_bit(z) << 3) | 7);
  int best = 0;
  double bestd = fabs(a - kE2M1[0]);
  for (int k = 1; k < 8; ++k) {
    double d = fabs(a - kE2M1[k]); /* exact: a < 6 is binary32, grid points are dyadic */
    if (d < bestd || (d == bestd && (k % 2) == 0)) {
      best = k;
      bestd = d;
    }
  }
  return (uint8_t)((sign_bit(z) << 3) | best);
}

/* Stochastic rounding ([P1] section 2d): between the two neighbouring grid
 * points lo <= |z| < hi, round up with probability equal to the fractional
 * distance f = (|z| - lo) / (hi - lo).  Reading used here: the decision takes
 * the top 22 bits u of the random word and the fraction truncated to 22 bits,
 * F = floor(f * 2^22), and rounds up iff u + F >= 2^22; so P(up) = F / 2^22,
 * which is f to within 2^-22.  |z| >= 6 gives 6; grid points are never moved. */
uint8_t orc_e2m1_sr(float z, uint32_t rword) {
  double a = fabs((double)z);
  int s = sign_bit(z);
  if (a >= 6.0) return (uint8_t)((s << 3) | 7);
  int k = 0;
  for (int i = 0; i < 8; ++i)
    if (kE2M1[i] <= a) k = i;
  double f = (a - kE2M1[k]) / (kE2M1[k + 1] - kE2M1[k]); /* exact: dyadic operands, power-of-two divisor */
  uint32_t F = (uint32_t)floor(f * 4194304.0);
  uint32_t u = rword >> 10;
  int up = (u + F) >= 4194304u;
  return (uint8_t)((s << 3) | (k + up));
}

float orc_e2m1_value(uint8_t code) {
  double v = kE2M1[code & 7];
  return (float)((code & 8) ? -v : v);
}

/* E4M3 (OCP "E4M3FN"): 1 sign, 4 exponent bits with bias 7, 3 mantissa bits;
 * subnormals m * 2^-9; largest finite value 448 = 0x7E; 0x7F is NaN. */
float orc_e4m3_value(uint8_t code) {
  int e = (code >> 3) & 15, m = code & 7;
  double v = (e == 0) ? ldexp((double)m, -9) : ldexp((double)(8 + m), e - 10);
  return (float)((code & 0x80) ? -v : v);
}

/* Round half to even to an integer, exactly (q is exact in binary64). */
static double rne_int(double q) {
  double fl = floor(q);
  double d = q - fl;
  if (d > 0.5) return fl + 1.0;
  if (d < 0.5) return fl;
  return (fmod(fl, 2.0) == 0.0) ? fl : fl + 1.0;
}

/* Encode r >= 0 as the nearest E4M3 value (ties to even mantissa), saturating
 * at 448: everything at or above 448, including +inf, gives 0x7E. */
uint8_t orc_e4m3_rne_sat(float r) {
  double x = (double)r;
  if (!(x < 448.0)) return 0x7E;
  if (x < ldexp(1.0, -6)) {
    /* subnormal binade: quantum 2^-9; n = 8 lands on 2^-6 = code 0x08 */
    double n = rne_int(x * 512.0);
    return (uint8_t)n;
  }
  int e2;
  frexp(x, &e2);
  int E = e2 - 1; /* x in [2^E, 2^(E+1)), E in [-6, 8] */
  double q = ldexp(x, 3 - E); /* in [8, 16) */
  double n = rne_int(q);
  if (n == 16.0) {
    n = 8.0;
    E += 1;
  }
  if (E > 8 || (E == 8 && n > 14.0)) return 0x7E;
  return (uint8_t)(((E + 7) << 3) | ((int)n - 8));
}

/* ------------------------------------------------------------------------ */
/* Philox-4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as   */
/* easy as 1, 2, 3", SC'11): ten rounds of two 32x32->64 multiplications with */
/* the published multipliers, the key bumped by the published Weyl constants  */
/* between rounds.                                                            */
/* ------------------------------------------------------------------------ */
void orc_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]) {
  const uint32_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u;
  const uint32_t W0 = 0x9E3779B9u, W1 = 0xBB67AE85u;
  uint32_t c0 = ctr[0], c1 = ctr[1], c2 = ctr[2], c3 = ctr[3];
  uint32_t k0 = key[0], k1 = key[1];
  for (int round = 0; round < 10; ++round) {
    if (round > 0) {
      k0 += W0;
      k1 += W1;
    }
    uint64_t p0 = (uint64_t)M0 * c0;
    uint64_t p1 = (uint64_t)M1 * c2;
    uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0;
    uint32_t n1 = (uint32_t)p1;
    uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
    uint32_t n3 = (uint32_t)p0;
    c0 = n0;
    c1 = n1;
    c2 = n2;
    c3 = n3;
  }
  out[0] = c0;
  out[1] = c1;
  out[2] = c2;
  out[3] = c3;
}

/* One 32-bit word per element: key = (seed low, seed high); counter =
 * (q low, q high, 0, 0) with q = idx / 4; the word is output (idx mod 4). */
uint32_t orc_sr_word(uint64_t seed, uint64_t idx) {
  uint64_t q = idx >> 2;
  uint32_t ctr[4] = {(uint32_t)q, (uint32_t)(q >> 32), 0u, 0u};
  uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
  uint32_t out[4];
  orc_philox4x32_10(ctr, key, out);
  return out[idx & 3];
}

/* Sign mask for the Hadamard transform: low 16 bits of word 0 at counter
 * (0, 0, 0, 1).  The stochastic-rounding stream always has counter word 3 = 0,
 * so the two streams never share a counter. */
uint32_t orc_rht_mask_from_seed(uint64_t seed) {
  uint32_t ctr[4] = {0u, 0u, 0u, 1u};
  uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
  uint32_t out[4];
  orc_philox4x32_10(ctr, key, out);
  return out[0] & 0xFFFFu;
}

/* ------------------------------------------------------------------------ */
/* 16-point random Hadamard transform ([P1] section 2b): y = H16 * D * x / 4  */
/* with H16 the Sylvester Hadamard matrix in natural order and D = diag(+-1). */
/* Stages h = 1, 2, 4, 8; in each, pairs (i, i+h) with (i & h) == 0 become    */
/* (fl(a+b), fl(a-b)); then every value is multiplied by 0.25 (exact).        */
/* ------------------------------------------------------------------------ */
void orc_rht16(const float* x, uint32_t mask, float* y) {
  float v[16];
  for (int i = 0; i < 16; ++i) v[i] = ((mask >> i) & 1u) ? -x[i] : x[i];
  for (int h = 1; h < 16; h <<= 1) {
    for (int i = 0; i < 16; ++i) {
      if (i & h) continue;
      float a = v[i], b = v[i + h];
      v[i] = a + b;
      v[i + h] = a - b;
    }
  }
  for (int i = 0; i < 16; ++i) y[i] = 0.25f * v[i];
}

/* ------------------------------------------------------------------------ */
/* Block quantization ([P2] "Core mechanism", "Adaptive block scaling")      */
/* ------------------------------------------------------------------------ */

/* Pairwise sum in index order: (t0+t1), (t2+t3), ..., then pairs of those. */
static float pairwise_sum(const float* t, int n) {
  if (n == 1) return t[0];
  int h = n / 2;
  float a = pairwise_sum(t, h);
  float b = pairwise_sum(t + h, h);
  return a + b;
}

/* One candidate: scale the block's max to T (6, or 4 for the 4/6 alternative).
 *   den = fl(T * s_t); r = fl(m_b / den) (0 if m_b or den is 0)
 *   sb  = E4M3(r);     d = fl(dec(sb) * s_t); e = fl(1 / d) (0 if d is 0 or 1/d overflows)
 *   z_i = fl(y_i * e); code_i = round(z_i)
 * Stochastic rounding draws element i's decision from its random word w_i:
 * the scale-to-6 candidate (and plain NVFP4) uses bits 31..10 of w_i, the
 * scale-to-4 candidate bits 30..9 (the word shifted left by one).  Both are
 * uniform 22-bit numbers, so each candidate's rounding is unbiased; the pages
 * fix only that the decision is random with the fractional distance as its
 * probability, not which bits of the element's word feed it.
 * With rule != NONE, the error against the values being quantized
 * ([P2] "Adaptive block scaling", step 2) is
 *   xh_i = fl(value(code_i) * d); eps_i = fl(y_i - xh_i)
 *   MSE: pairwise sum of fl(eps_i * eps_i); MAE: pairwise sum of |eps_i|; MAXERR: max |eps_i|. */
static void candidate(const float* y, int n, float m_b, float T, float s_t, int rule, int sr,
                      const uint32_t* rwords, uint8_t* codes, uint8_t* sb_out, float* err) {
  float den = T * s_t;
  float r = (m_b == 0.0f || den == 0.0f) ? 0.0f : m_b / den;
  uint8_t sb = orc_e4m3_rne_sat(r);
  float d = orc_e4m3_value(sb) * s_t;
  float e = 0.0f;
  if (d != 0.0f) {
    e = 1.0f / d;
    if (isinf(e)) e = 0.0f;
  }
  for (int i = 0; i < n; ++i) {
    float z = y[i] * e;
    if (!sr) codes[i] = orc_e2m1_rne(z);
    else codes[i] = orc_e2m1_sr(z, T == 4.0f ? rwords[i] << 1 : rwords[i]);
  }
  *sb_out = sb;
  *err = 0.0f;
  if (rule == ORC_RULE_NONE) return;
  float t[256];
  float mx = 0.0f;
  for (int i = 0; i < n; ++i) {
    float xh = orc_e2m1_value(codes[i]) * d;
    float eps = y[i] - xh;
    float ae = fabsf(eps);
    if (rule == ORC_RULE_MSE) t[i] = eps * eps;
    else t[i] = ae;
    if (ae > mx) mx = ae;
  }
  *err = (rule == ORC_RULE_MAXERR) ? mx : pairwise_sum(t, n);
}

void orc_quantize_block(const float* y, int n, float s_t, int rule, int sr, const uint32_t* rwords,
                        uint8_t* codes, uint8_t* scale, uint8_t* chose4, float* err) {
  float m_b = 0.0f;
  for (int i = 0; i < n; ++i) {
    float a = fabsf(y[i]);
    if (a > m_b) m_b = a;
  }
  uint8_t c6[256], sb6;
  float e6;
  candidate(y, n, m_b, 6.0f, s_t, rule, sr, rwords, c6, &sb6, &e6);
  err[0] = e6;
  err[1] = 0.0f;
  *chose4 = 0;
  if (rule != ORC_RULE_NONE) {
    uint8_t c4[256], sb4;
    float e4;
    candidate(y, n, m_b, 4.0f, s_t, rule, sr, rwords, c4, &sb4, &e4);
    err[1] = e4;
    if (e4 < e6) { /* strict: a tie keeps the standard scale-to-6 block */
      memcpy(codes, c4, (size_t)n);
      *scale = sb4;
      *chose4 = 1;
      return;
    }
  }
  memcpy(codes, c6, (size_t)n);
  *scale = sb6;
}

/* ------------------------------------------------------------------------ */
/* Tensor level                                                               */
/* ------------------------------------------------------------------------ */

static float load_elem(const void* x, int dtype, int64_t i) {
  if (dtype == ORC_IN_F32) return ((const float*)x)[i];
  return orc_bf16_to_f32(((const uint16_t*)x)[i]);
}

/* The per-tensor amax behind the FP32 tensor scale ([P2] "Implementation
 * details").  With the transform on, it is the amax of the transformed tensor. */
float orc_amax(const void* x, int dtype, int64_t rows, int64_t cols, int rht, uint32_t mask) {
  float A = 0.0f;
  if (!rht) {
    for (int64_t i = 0; i < rows * cols; ++i) {
      float a = fabsf(load_elem(x, dtype, i));
      if (a > A) A = a;
    }
    return A;
  }
  float in[16], out[16];
  for (int64_t r = 0; r < rows; ++r) {
    for (int64_t j = 0; j < cols / 16; ++j) {
      for (int k = 0; k < 16; ++k) in[k] = load_elem(x, dtype, r * cols + j * 16 + k);
      orc_rht16(in, mask, out);
      for (int k = 0; k < 16; ++k) {
        float a = fabsf(out[k]);
        if (a > A) A = a;
      }
    }
  }
  return A;
}

/* S_t = fl(A / fl(6 * cap)); the block scale maps a block's max to
 * 6 * dec(sb) * S_t, so the largest block lands on the E4M3 value `cap`. */
float orc_tensor_scale(float amax, float cap) {
  float c6 = 6.0f * cap;
  return amax / c6;
}

typedef struct {
  const void* x;
  int dtype;
  int64_t rows, cols, r0, r1;
  const orc_config* cfg;
  float s_t;
  uint8_t *codes_row, *scales_row, *codes_col, *scales_col, *pick_row, *pick_col;
} band_job;

static void put_nibble(uint8_t* base, int64_t byte, int hi, uint8_t code) {
  if (hi) base[byte] = (uint8_t)((base[byte] & 0x0F) | (code << 4));
  else base[byte] = (uint8_t)((base[byte] & 0xF0) | (code & 0x0F));
}

static void fill_words(const orc_config* cfg, const int64_t* idx, int n, uint32_t* w) {
  for (int i = 0; i < n; ++i) w[i] = cfg->sr ? orc_sr_word(cfg->sr_seed, (uint64_t)idx[i]) : 0u;
}

/* Rows [r0, r1) of the tensor; r0 and r1 are multiples of 16 whenever a
 * column copy or 2D tiles are requested. */
static void quantize_band(const band_job* J) {
  const orc_config* cfg = J->cfg;
  const int64_t M = J->rows, N = J->cols;
  float y[256];
  int64_t idx[256];
  uint32_t w[256];
  uint8_t codes[256], sb, ch;
  float err[2];

  if (cfg->block_2d) {
    /* [P1] section 2c: one scale per 16x16 tile, shared by both orientations. */
    for (int64_t ti = J->r0 / 16; ti < J->r1 / 16; ++ti) {
      for (int64_t tj = 0; tj < N / 16; ++tj) {
        for (int i = 0; i < 16; ++i)
          for (int j = 0; j < 16; ++j) {
            int64_t r = ti * 16 + i, c = tj * 16 + j;
            y[i * 16 + j] = load_elem(J->x, J->dtype, r * N + c);
            idx[i * 16 + j] = (cfg->row_offset + r) * N + c;
          }
        fill_words(cfg, idx, 256, w);
        orc_quantize_block(y, 256, J->s_t, cfg->rule, cfg->sr, w, codes, &sb, &ch, err);
        if (cfg->emit_row) {
          J->scales_row[ti * (N / 16) + tj] = sb;
          if (J->pick_row) J->pick_row[ti * (N / 16) + tj] = ch;
          for (int i = 0; i < 16; ++i)
            for (int j = 0; j < 16; ++j) {
              int64_t r = ti * 16 + i, c = tj * 16 + j;
              put_nibble(J->codes_row, r * (N / 2) + c / 2, (int)(c & 1), codes[i * 16 + j]);
            }
        }
        if (cfg->emit_col) {
          J->scales_col[tj * (M / 16) + ti] = sb;
          if (J->pick_col) J->pick_col[tj * (M / 16) + ti] = ch;
          for (int i = 0; i < 16; ++i)
            for (int j = 0; j < 16; ++j) {
              int64_t r = ti * 16 + i, c = tj * 16 + j;
              put_nibble(J->codes_col, c * (M / 2) + r / 2, (int)(r & 1), codes[i * 16 + j]);
            }
        }
      }
    }
    return;
  }

  if (cfg->emit_row) {
    float in[16];
    for (int64_t r = J->r0; r < J->r1; ++r) {
      for (int64_t j = 0; j < N / 16; ++j) {
        for (int k = 0; k < 16; ++k) {
          in[k] = load_elem(J->x, J->dtype, r * N + j * 16 + k);
          idx[k] = (cfg->row_offset + r) * N + j * 16 + k;
        }
        if (cfg->rht) orc_rht16(in, cfg->rht_mask, y);
        else memcpy(y, in, sizeof(in));
        fill_words(cfg, idx, 16, w);
        orc_quantize_block(y, 16, J->s_t, cfg->rule, cfg->sr, w, codes, &sb, &ch, err);
        J->scales_row[r * (N / 16) + j] = sb;
        if (J->pick_row) J->pick_row[r * (N / 16) + j] = ch;
        for (int k = 0; k < 16; ++k) put_nibble(J->codes_row, r * (N / 2) + (j * 16 + k) / 2, k & 1, codes[k]);
      }
    }
  }
  if (cfg->emit_col) {
    /* [P1] section 2c: the backward pass needs the column orientation; here
     * each column is cut into 16x1 blocks of the same values (same S_t). */
    for (int64_t c = 0; c < N; ++c) {
      for (int64_t i = J->r0 / 16; i < J->r1 / 16; ++i) {
        for (int k = 0; k < 16; ++k) {
          int64_t r = i * 16 + k;
          y[k] = load_elem(J->x, J->dtype, r * N + c);
          idx[k] = (cfg->row_offset + r) * N + c;
        }
        fill_words(cfg, idx, 16, w);
        orc_quantize_block(y, 16, J->s_t, cfg->rule, cfg->sr, w, codes, &sb, &ch, err);
        J->scales_col[c * (M / 16) + i] = sb;
        if (J->pick_col) J->pick_col[c * (M / 16) + i] = ch;
        for (int k = 0; k < 16; ++k) put_nibble(J->codes_col, c * (M / 2) + (i * 16 + k) / 2, k & 1, codes[k]);
      }
    }
  }
}

static void* band_thread(void* arg) {
  quantize_band((const band_job*)arg);
  return NULL;
}

int orc_quantize(const void* x, int dtype, int64_t rows, int64_t cols, const orc_config* cfg, float amax,
                 uint8_t* codes_row, uint8_t* scales_row, uint8_t* codes_col, uint8_t* scales_col,
                 float* tensor_scale, uint8_t* pick_row, uint8_t* pick_col, int nthreads) {
  if (rows < 0 || cols < 0) return 1;
  if (dtype != ORC_IN_BF16 && dtype != ORC_IN_F32) return 1;
  if (cfg->cap != 448.0f && cfg->cap != 256.0f) return 1;
  if (cfg->rule < ORC_RULE_NONE || cfg->rule > ORC_RULE_MAXERR) return 1;
  if (cols % 16) return 1;
  int need16 = cfg->block_2d || cfg->emit_col;
  if (need16 && rows % 16) return 1;
  if (cfg->rht && (cfg->block_2d || cfg->emit_col)) return 1;
  float s_t = orc_tensor_scale(amax, cfg->cap);
  if (tensor_scale) *tensor_scale = s_t;
  if (rows == 0 || cols == 0) return 0;

  if (nthreads < 1) nthreads = 1;
  int64_t groups = (rows + 15) / 16; /* bands are whole 16-row groups */
  if (nthreads > groups) nthreads = (int)groups;
  band_job* jobs = (band_job*)calloc((size_t)nthreads, sizeof(band_job));
  pthread_t* th = (pthread_t*)calloc((size_t)nthreads, sizeof(pthread_t));
  if (!jobs || !th) {
    free(jobs);
    free(th);
    return 2;
  }
  for (int t = 0; t < nthreads; ++t) {
    int64_t g0 = groups * t / nthreads, g1 = groups * (t + 1) / nthreads;
    band_job J = {x, dtype, rows, cols, g0 * 16, g1 * 16 < rows ? g1 * 16 : rows, cfg, s_t,
                  codes_row, scales_row, codes_col, scales_col, pick_row, pick_col};
    jobs[t] = J;
  }
  if (nthreads == 1) {
    quantize_band(&jobs[0]);
  } else {
    for (int t = 0; t < nthreads; ++t) pthread_create(&th[t], NULL, band_thread, &jobs[t]);
    for (int t = 0; t < nthreads; ++t) pthread_join(th[t], NULL);
  }
  free(jobs);
  free(th);
  return 0;
}

/* x_hat = fl(value(code) * fl(dec(sb) * S_t)): the same d as the block's
 * chosen candidate, so this reproduces xh_i of the 4/6 error exactly. */
void orc_dequantize(const uint8_t* codes, const uint8_t* scales, float tensor_scale, int64_t rows, int64_t cols,
                    int block_2d, float* out) {
  for (int64_t r = 0; r < rows; ++r) {
    for (int64_t c = 0; c < cols; ++c) {
      uint8_t byte = codes[r * (cols / 2) + c / 2];
      uint8_t code = (c & 1) ? (uint8_t)(byte >> 4) : (uint8_t)(byte & 15);
      uint8_t sb = block_2d ? scales[(r / 16) * (cols / 16) + c / 16] : scales[r * (cols / 16) + c / 16];
      float d = orc_e4m3_value(sb) * tensor_scale;
      out[r * cols + c] = orc_e2m1_value(code) * d;
    }
  }
}

/* ------------------------------------------------------------------------ */
/* Error analysis by scaled value ([P2] "Problem statement")                  */
/* ------------------------------------------------------------------------ */

/* Nearest E2M1 magnitude to q >= 0 (binary64), ties to the even grid index. */
static double e2m1_nearest64(double q) {
  if (q >= 6.0) return 6.0;
  int best = 0;
  double bestd = fabs(q - kE2M1[0]);
  for (int k = 1; k < 8; ++k) {
    double d = fabs(q - kE2M1[k]);
    if (d < bestd || (d == bestd && (k % 2) == 0)) {
      best = k;
      bestd = d;
    }
  }
  return kE2M1[best];
}

/* Per block: the quantized path exactly as orc_quantize computes it (RNE), and
 * a reference with an unquantized scale: the block max maps exactly to T (the
 * candidate the block chose), v* = nearest-even E2M1 of q = fl64(T*|y| / m_b),
 * xh* = fl64(v* * m_b / T) with the sign of y.  Each element lands in the bin of
 * its scaled value |z|, z = fl(y * e); per bin the element count, the sum of
 * eps^2 (eps = fl(y - fl(v * d))) and the sum of eps*^2 (eps* = fl64(y - xh*))
 * are accumulated in binary64 in element order. */
static void err_block(const float* y, int n, float s_t, int rule, float inv_w, int nbins, double* stats) {
  uint8_t codes[256], sb, ch;
  float err[2];
  orc_quantize_block(y, n, s_t, rule, 0, NULL, codes, &sb, &ch, err);
  const double T = ch ? 4.0 : 6.0;
  float d = orc_e4m3_value(sb) * s_t;
  float e = 0.0f;
  if (d != 0.0f) {
    e = 1.0f / d;
    if (isinf(e)) e = 0.0f;
  }
  float m_b = 0.0f;
  for (int i = 0; i < n; ++i)
    if (fabsf(y[i]) > m_b) m_b = fabsf(y[i]);
  for (int i = 0; i < n; ++i) {
    float z = y[i] * e;
    int b = (int)floorf(fabsf(z) * inv_w); /* exact: inv_w is a power of two */
    if (b > nbins - 1) b = nbins - 1;
    float xh = orc_e2m1_value(codes[i]) * d;
    float eps = y[i] - xh;
    double xs = 0.0;
    if (m_b != 0.0f) {
      double q = (T * fabs((double)y[i])) / (double)m_b;
      xs = (e2m1_nearest64(q) * (double)m_b) / T;
    }
    double eps_s = (double)y[i] - copysign(xs, (double)y[i]);
    stats[b] += 1.0;
    stats[nbins + b] += (double)eps * (double)eps;
    stats[2 * nbins + b] += eps_s * eps_s;
  }
}

int orc_error_stats(const void* x, int dtype, int64_t rows, int64_t cols, const orc_config* cfg, float amax,
                    float bin_width, int nbins, double* stats) {
  if (rows < 0 || cols < 0 || cols % 16 || rows % 16 || nbins < 1 || nbins > 64) return 1;
  if (cfg->sr || (cfg->rht && cfg->block_2d)) return 1;
  int eb;
  if (!(bin_width > 0.0f) || frexpf(bin_width, &eb) != 0.5f) return 1; /* a power of two */
  const float inv_w = 1.0f / bin_width;
  const float s_t = orc_tensor_scale(amax, cfg->cap);
  memset(stats, 0, sizeof(double) * 3 * (size_t)nbins);
  float y[256];
  if (cfg->block_2d) {
    for (int64_t tr = 0; tr < rows / 16; ++tr)
      for (int64_t tc = 0; tc < cols / 16; ++tc) {
        for (int i = 0; i < 16; ++i)
          for (int j = 0; j < 16; ++j) y[i * 16 + j] = load_elem(x, dtype, (tr * 16 + i) * cols + tc * 16 + j);
        err_block(y, 256, s_t, cfg->rule, inv_w, nbins, stats);
      }
    return 0;
  }
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t j = 0; j < cols / 16; ++j) {
      for (int k = 0; k < 16; ++k) y[k] = load_elem(x, dtype, r * cols + j * 16 + k);
      if (cfg->rht) {
        float t[16];
        orc_rht16(y, cfg->rht_mask, t);
        memcpy(y, t, sizeof(t));
      }
      err_block(y, 16, s_t, cfg->rule, inv_w, nbins, stats);
    }
  return 0;
}

/* ------------------------------------------------------------------------ */
/* The consumer: a GEMM on block-scaled FP4 operands                          */
/* ------------------------------------------------------------------------ */

/* The value an operand element encodes, exactly (binary64 holds it):
 * NVFP4: v(code) * dec(sb), the tensor scale applied once to the whole product;
 * MXFP4: v(code) * 2^(sc - 127). */
static double nv_elem(const uint8_t* codes, const uint8_t* scales, int block_2d, int64_t r, int64_t k, int64_t K) {
  uint8_t byte = codes[r * (K / 2) + k / 2];
  uint8_t c = (k & 1) ? (uint8_t)(byte >> 4) : (uint8_t)(byte & 15);
  uint8_t sb = block_2d ? scales[(r / 16) * (K / 16) + k / 16] : scales[r * (K / 16) + k / 16];
  return (double)orc_e2m1_value(c) * (double)orc_e4m3_value(sb);
}

static double mx_elem(const uint8_t* codes, const uint8_t* scales, int64_t r, int64_t k, int64_t K) {
  uint8_t byte = codes[r * (K / 2) + k / 2];
  uint8_t c = (k & 1) ? (uint8_t)(byte >> 4) : (uint8_t)(byte & 15);
  return (double)orc_e2m1_value(c) * (double)orc_e8m0_value(scales[r * (K / 32) + k / 32]);
}

int orc_gemm_fp4(int mx, const uint8_t* a_codes, const uint8_t* a_scales, float a_ts, int a_2d, const uint8_t* b_codes,
                 const uint8_t* b_scales, float b_ts, int b_2d, int64_t M, int64_t N, int64_t K, float* c,
                 double* c_abs) {
  if (M < 0 || N < 0 || K < 0 || K % (mx ? 32 : 16)) return 1;
  if (!mx && ((a_2d && M % 16) || (b_2d && N % 16))) return 1;
  const double ts = mx ? 1.0 : (double)a_ts * (double)b_ts;
  for (int64_t m = 0; m < M; ++m) {
    for (int64_t n = 0; n < N; ++n) {
      double acc = 0.0, aacc = 0.0;
      for (int64_t k = 0; k < K; ++k) {
        double a = mx ? mx_elem(a_codes, a_scales, m, k, K) : nv_elem(a_codes, a_scales, a_2d, m, k, K);
        double b = mx ? mx_elem(b_codes, b_scales, n, k, K) : nv_elem(b_codes, b_scales, b_2d, n, k, K);
        acc += a * b; /* each product is exact in binary64 */
        aacc += fabs(a * b);
      }
      c[m * N + n] = (float)(acc * ts);
      if (c_abs) c_abs[m * N + n] = aacc * fabs(ts);
    }
  }
  return 0;
}

/* ------------------------------------------------------------------------ */
/* MXFP4: 32-element blocks with power-of-two (E8M0) scales                   */
/* ------------------------------------------------------------------------ */

/* E8M0: 2^(code - 127); the code 255 is NaN in the MX specification. */
float orc_e8m0_value(uint8_t code) { return code == 255 ? NAN : (float)ldexp(1.0, (int)code - 127); }

/* Shared exponent of a block: floor(log2(m)) - 2, so that the block max
 * scales into [4, 8); clamped to the E8M0 range [-127, 127]. */
uint8_t orc_mx_scale_code(float block_max) {
  if (block_max == 0.0f) return 0;  /* 2^-127: every element becomes +-0 */
  int e2;
  frexp((double)block_max, &e2); /* block_max = f * 2^e2, f in [0.5, 1) */
  int e = (e2 - 1) - 2;
  if (e < -127) e = -127;
  if (e > 127) e = 127;
  return (uint8_t)(e + 127);
}

/* One 32-element block: y[k] is element k, idx[k] its flat index (for the
 * stochastic-rounding word).  Writes 16 code bytes and returns the scale code. */
static uint8_t mx_block(const float* y, const uint64_t* idx, int sr, uint64_t sr_seed, uint8_t* codes) {
  float m = 0.0f;
  for (int k = 0; k < 32; ++k) {
    float a = fabsf(y[k]);
    if (a > m) m = a;
  }
  uint8_t sc = orc_mx_scale_code(m);
  for (int k = 0; k < 32; ++k) {
    /* y / 2^e: exact in binary64, then one rounding to binary32 (only values far
     * below the E2M1 grid can lose bits there) */
    float z = (float)ldexp((double)y[k], 127 - (int)sc);
    uint8_t c = sr ? orc_e2m1_sr(z, orc_sr_word(sr_seed, idx[k])) : orc_e2m1_rne(z);
    put_nibble(codes, k / 2, k & 1, c);
  }
  return sc;
}

int orc_mxfp4_quantize(const void* x, int dtype, int64_t rows, int64_t cols, int emit_row, int emit_col, int sr,
                       uint64_t sr_seed, int64_t row_offset, uint8_t* codes_row, uint8_t* scales_row,
                       uint8_t* codes_col, uint8_t* scales_col) {
  if (rows < 0 || cols < 0) return 1;
  if (emit_row && cols % 32) return 1;
  if (emit_col && rows % 32) return 1;
  if (dtype != ORC_IN_BF16 && dtype != ORC_IN_F32) return 1;
  float y[32];
  uint64_t idx[32];
  if (emit_row) {
    for (int64_t r = 0; r < rows; ++r) {
      for (int64_t j = 0; j < cols / 32; ++j) {
        for (int k = 0; k < 32; ++k) {
          y[k] = load_elem(x, dtype, r * cols + j * 32 + k);
          idx[k] = (uint64_t)((row_offset + r) * cols + j * 32 + k);
        }
        scales_row[r * (cols / 32) + j] = mx_block(y, idx, sr, sr_seed, codes_row + r * (cols / 2) + j * 16);
      }
    }
  }
  if (emit_col) {
    /* the column copy: blocks of 32 rows of one column; the copy is stored
     * transposed ([cols][rows/2]), and each element keeps its own random word */
    for (int64_t c = 0; c < cols; ++c) {
      for (int64_t j = 0; j < rows / 32; ++j) {
        for (int k = 0; k < 32; ++k) {
          y[k] = load_elem(x, dtype, (j * 32 + k) * cols + c);
          idx[k] = (uint64_t)((row_offset + j * 32 + k) * cols + c);
        }
        scales_col[c * (rows / 32) + j] = mx_block(y, idx, sr, sr_seed, codes_col + c * (rows / 2) + j * 16);
      }
    }
  }
  return 0;
}

void orc_mxfp4_dequantize(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t cols, float* out) {
  for (int64_t r = 0; r < rows; ++r) {
    for (int64_t c = 0; c < cols; ++c) {
      uint8_t byte = codes[r * (cols / 2) + c / 2];
      uint8_t code = (c & 1) ? (uint8_t)(byte >> 4) : (uint8_t)(byte & 15);
      uint8_t sc = scales[r * (cols / 32) + c / 32];
      out[r * cols + c] = (float)((double)orc_e2m1_value(code) * (double)orc_e8m0_value(sc));
    }
  }
}

/* ------------------------------------------------------------------------ */
/* Batch wrappers (so the pins can sweep millions of values cheaply)          */
/* ------------------------------------------------------------------------ */
void orc_e2m1_rne_n(const float* z, int64_t n, uint8_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_e2m1_rne(z[i]);
}
void orc_e2m1_sr_n(const float* z, const uint32_t* w, int64_t n, uint8_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_e2m1_sr(z[i], w[i]);
}
void orc_e4m3_rne_sat_n(const float* r, int64_t n, uint8_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_e4m3_rne_sat(r[i]);
}
void orc_sr_words_n(uint64_t seed, const uint64_t* idx, int64_t n, uint32_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_sr_word(seed, idx[i]);
}
void orc_philox_n(const uint32_t* ctr, const uint32_t* key, int64_t n, uint32_t* out) {
  for (int64_t i = 0; i < n; ++i) orc_philox4x32_10(ctr + 4 * i, key + 2 * i, out + 4 * i);
}
