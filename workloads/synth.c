/*
 * synth.c -- seeded synthetic input tensors for the NVFP4 quantization workloads.
 *
 * Holds no quantization arithmetic: it only draws numbers.  Both the GPU tests
 * and the CPU oracle consume the bytes it writes, so the two sides always see
 * identical inputs.
 *
 * Randomness is counter based: u(seed, stream, i) is the SplitMix64 output
 * function (Steele, Lea, Flood, "Fast splittable pseudorandom number
 * generators", OOPSLA 2014) applied to seed ^ (stream << 56) + (i + 1) * gamma,
 * mapped to a double in (0, 1).  Normals use the Box-Muller transform in double.
 * Values are rounded to binary32 and, for bf16 tensors, to bf16 (nearest even).
 *
 * Recipes (kind):
 *   1  fp32, N(0,1); each element with probability 0.01 multiplied by 50
 *   2  bf16, N(0,1); floor(0.5% of cols) (at least 1) columns, picked by a
 *      seeded Fisher-Yates shuffle, multiplied by 20 (channel outliers)
 *   3  bf16, N(0, sigma=0.02); each element with probability 0.001 multiplied by 30
 *   4  bf16, Student-t with 3 degrees of freedom, times 1e-3:
 *      t = Z0 / sqrt((Z1^2 + Z2^2 + Z3^2) / 3)
 *   5  bf16, per element: with probability 0.02 N(0, sigma=20), else N(0,1)
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

static uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

static double unif(uint64_t seed, uint64_t stream, uint64_t i) {
  uint64_t z = mix64((seed ^ (stream << 56)) + (i + 1) * 0x9E3779B97F4A7C15ull);
  return ((double)(z >> 11) + 0.5) * (1.0 / 9007199254740992.0);
}

static double normal(uint64_t seed, uint64_t stream, uint64_t i) {
  double u1 = unif(seed, stream, 2 * i), u2 = unif(seed, stream, 2 * i + 1);
  return sqrt(-2.0 * log(u1)) * cos(6.283185307179586 * u2);
}

static uint16_t f32_to_bf16(float f) {
  uint32_t b;
  memcpy(&b, &f, 4);
  b += 0x7FFFu + ((b >> 16) & 1u);
  return (uint16_t)(b >> 16);
}

typedef struct {
  int kind;
  int64_t rows, cols, r0, r1;
  uint64_t seed;
  void* out;
  const uint8_t* col_flag;
} job_t;

static double draw(const job_t* J, int64_t r, int64_t c) {
  uint64_t i = (uint64_t)(r * J->cols + c);
  uint64_t s = J->seed;
  switch (J->kind) {
    case 1: {
      double v = normal(s, 0, i);
      return unif(s, 2, i) < 0.01 ? v * 50.0 : v;
    }
    case 2: {
      double v = normal(s, 0, i);
      return J->col_flag[c] ? v * 20.0 : v;
    }
    case 3: {
      double v = 0.02 * normal(s, 0, i);
      return unif(s, 2, i) < 0.001 ? v * 30.0 : v;
    }
    case 4: {
      double z0 = normal(s, 0, i), z1 = normal(s, 4, i), z2 = normal(s, 5, i), z3 = normal(s, 6, i);
      return 1e-3 * z0 / sqrt((z1 * z1 + z2 * z2 + z3 * z3) / 3.0);
    }
    case 5: {
      double v = normal(s, 0, i);
      return unif(s, 2, i) < 0.02 ? 20.0 * v : v;
    }
  }
  return 0.0;
}

static void* run(void* arg) {
  const job_t* J = (const job_t*)arg;
  for (int64_t r = J->r0; r < J->r1; ++r) {
    for (int64_t c = 0; c < J->cols; ++c) {
      float f = (float)draw(J, r, c);
      if (J->kind == 1) ((float*)J->out)[r * J->cols + c] = f;
      else ((uint16_t*)J->out)[r * J->cols + c] = f32_to_bf16(f);
    }
  }
  return NULL;
}

/* out: rows*cols float32 (kind 1) or uint16 bf16 patterns (kinds 2-5).
 * Returns 0 on success. */
int synth_generate(int kind, int64_t rows, int64_t cols, uint64_t seed, void* out, int nthreads) {
  if (kind < 1 || kind > 5 || rows < 0 || cols < 0) return 1;
  uint8_t* flag = NULL;
  if (kind == 2 && cols > 0) {
    int64_t k = (int64_t)floor(0.005 * (double)cols);
    if (k < 1) k = 1;
    int64_t* perm = (int64_t*)malloc((size_t)cols * sizeof(int64_t));
    flag = (uint8_t*)calloc((size_t)cols, 1);
    if (!perm || !flag) {
      free(perm);
      free(flag);
      return 2;
    }
    for (int64_t c = 0; c < cols; ++c) perm[c] = c;
    for (int64_t c = cols - 1; c > 0; --c) { /* Fisher-Yates, stream 3 */
      int64_t j = (int64_t)(unif(seed, 3, (uint64_t)c) * (double)(c + 1));
      if (j > c) j = c;
      int64_t t = perm[c];
      perm[c] = perm[j];
      perm[j] = t;
    }
    for (int64_t q = 0; q < k; ++q) flag[perm[q]] = 1;
    free(perm);
  }
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  if (rows < nthreads) nthreads = rows > 0 ? (int)rows : 1;
  pthread_t th[256];
  job_t jobs[256];
  for (int t = 0; t < nthreads; ++t) {
    job_t J = {kind, rows, cols, rows * t / nthreads, rows * (t + 1) / nthreads, seed, out, flag};
    jobs[t] = J;
  }
  if (nthreads == 1) {
    run(&jobs[0]);
  } else {
    for (int t = 0; t < nthreads; ++t) pthread_create(&th[t], NULL, run, &jobs[t]);
    for (int t = 0; t < nthreads; ++t) pthread_join(th[t], NULL);
  }
  free(flag);
  return 0;
}
