/*
 * oracle_driver.c -- runs every entry point of the oracle (oracle/oracle.c)
 * on seeded random inputs and edge cases, with every buffer allocated at
 * its exact size, so that a build under AddressSanitizer and
 * UndefinedBehaviorSanitizer (tests/sanitize/build.py) reports any
 * out-of-bounds access, leak or undefined operation in the host C code.
 * Exit status 0 when every call returned what its contract says.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "oracle.h"

static uint64_t state = 0x9E3779B97F4A7C15ull;
static uint64_t next_u64(void) {  /* SplitMix64 */
  uint64_t z = (state += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}
static double uniform(void) { return (double)(next_u64() >> 11) * 0x1p-53; }

static int failures = 0;
#define EXPECT(cond, what)                                      \
  do {                                                          \
    if (!(cond)) {                                              \
      fprintf(stderr, "FAILED: %s (line %d)\n", what, __LINE__); \
      ++failures;                                               \
    }                                                           \
  } while (0)

/* rows x stride 16-bit values of N(0, std) (Box-Muller), encoded. */
static uint16_t *rand16(int dtype, int64_t rows, int64_t stride, double std) {
  uint16_t *p = malloc((size_t)(rows * stride) * sizeof(uint16_t));
  for (int64_t i = 0; i < rows * stride; ++i) {
    const double u1 = uniform() + 0x1p-60, u2 = uniform();
    p[i] = orc_encode16(dtype, std * sqrt(-2.0 * log(u1)) * cos(6.283185307179586 * u2));
  }
  return p;
}

static uint8_t *rand_codes(int64_t n) {
  uint8_t *p = malloc((size_t)n);
  for (int64_t i = 0; i < n; ++i) {
    uint8_t c = (uint8_t)next_u64();
    p[i] = (c & 0x7F) == 0x7F ? 0 : c;  /* no NaN codes */
  }
  return p;
}

static void norm_case(int dtype, int64_t rows, int64_t hidden, int64_t stride, int fused,
                      int with_w, int mode, int64_t var) {
  uint16_t *x = rand16(dtype, rows, stride, 1.0);
  uint16_t *r = fused ? rand16(dtype, rows, stride, 1.0) : NULL;
  uint16_t *w = with_w ? rand16(dtype, 1, hidden, 0.1) : NULL;
  uint16_t *r16 = malloc((size_t)(rows * hidden) * 2 + 1);
  double *y = malloc((size_t)(rows * hidden) * sizeof(double) + 1);
  uint16_t *y16 = malloc((size_t)(rows * hidden) * 2 + 1);
  uint8_t *q = malloc((size_t)(rows * hidden) + 1);
  float *sc = malloc((size_t)rows * sizeof(float) + 1);
  const int rc = var ? orc_add_rmsnorm_var(dtype, rows, hidden, var, x, stride, r, stride, w,
                                           1e-6f, r16, y, y16, mode, 0.05f, q, sc)
                     : orc_add_rmsnorm(dtype, rows, hidden, x, stride, r, stride, w, 1e-6f,
                                       r16, y, y16, mode, 0.05f, q, sc);
  EXPECT(rc == 0, "orc_add_rmsnorm");
  for (int64_t i = 0; i < rows * hidden; ++i) EXPECT(!isnan(y[i]), "finite y");
  free(x); free(r); free(w); free(r16); free(y); free(y16); free(q); free(sc);
}

int main(void) {
  /* codecs: every 16-bit pattern round-trips (NaNs excepted), every e4m3 code */
  for (int dt = 0; dt < 2; ++dt) {
    for (uint32_t b = 0; b < 65536; ++b) {
      const double v = orc_decode16(dt, (uint16_t)b);
      if (!isnan(v)) EXPECT(orc_encode16(dt, v) == (uint16_t)b, "16-bit round trip");
    }
  }
  for (int c = 0; c < 256; ++c) {
    const double v = orc_e4m3_decode((uint8_t)c);
    if (!isnan(v)) EXPECT(orc_e4m3_encode(v) == (uint8_t)c || v == 0.0, "e4m3 round trip");
  }
  EXPECT(orc_e4m3_encode(1e30) == 0x7E, "saturation");
  EXPECT(orc_e4m3_encode(NAN) == 0x7F, "NaN code");

  /* residual add */
  {
    const int64_t n = 1000;
    uint16_t *x = rand16(ORC_BF16, 1, n, 1.0), *r = rand16(ORC_BF16, 1, n, 1.0);
    uint16_t *o = malloc((size_t)n * 2);
    EXPECT(orc_residual16(ORC_BF16, n, x, r, o) == 0, "orc_residual16");
    EXPECT(orc_residual16(ORC_BF16, -1, x, r, o) == 1, "orc_residual16 n < 0");
    free(x); free(r); free(o);
  }

  /* norm: every mode, both dtypes, plain / fused, with and without weight,
     ragged and padded rows, one-channel rows, variance-size override */
  const int64_t shapes[][3] = {{5, 1, 1}, {3, 7, 9}, {4, 64, 64}, {2, 1000, 1024}, {1, 4096, 4096}};
  for (int s = 0; s < 5; ++s)
    for (int dt = 0; dt < 2; ++dt)
      for (int fused = 0; fused < 2; ++fused)
        for (int mode = -1; mode <= 1; ++mode)
          norm_case(dt, shapes[s][0], shapes[s][1], shapes[s][2], fused, (s + mode) & 1, mode, 0);
  norm_case(ORC_BF16, 3, 1000, 1000, 1, 1, ORC_FP8_DYNAMIC, 300);
  norm_case(ORC_FP16, 2, 64, 80, 0, 0, ORC_FP8_NONE, 64);
  norm_case(ORC_BF16, 0, 64, 64, 1, 1, ORC_FP8_NONE, 0);  /* no rows */
  {
    uint16_t x[4] = {0};
    double y[4];
    EXPECT(orc_add_rmsnorm(2, 1, 4, x, 4, NULL, 4, NULL, 1e-6f, NULL, y, NULL, -1, 0, NULL, NULL) == -1,
           "unknown dtype refused");
    EXPECT(orc_add_rmsnorm(0, 1, 4, x, 3, NULL, 4, NULL, 1e-6f, NULL, y, NULL, -1, 0, NULL, NULL) == -1,
           "stride < hidden refused");
    EXPECT(orc_add_rmsnorm_var(0, 1, 4, 5, x, 4, NULL, 4, NULL, 1e-6f, NULL, y, NULL, -1, 0, NULL,
                               NULL) == -1, "variance size > hidden refused");
  }

  /* all-reduce step over 1..8 parts */
  for (int np = 1; np <= 8; ++np) {
    const int64_t rows = 3, hidden = 130, stride = 136;
    const uint16_t *parts[8];
    uint16_t *owned[8];
    for (int g = 0; g < np; ++g) parts[g] = owned[g] = rand16(ORC_BF16, rows, stride, 0.5);
    uint16_t *x16 = malloc((size_t)(rows * hidden) * 2);
    EXPECT(orc_sum_parts16(ORC_BF16, np, parts, stride, rows, hidden, x16) == 0, "orc_sum_parts16");
    for (int g = 0; g < np; ++g) free(owned[g]);
    free(x16);
  }

  /* SwiGLU: every mode, split tensors with their own strides */
  for (int mode = -1; mode <= 1; ++mode) {
    const int64_t rows = 4, d = 333;
    uint16_t *gate = rand16(ORC_FP16, rows, d + 5, 2.0), *up = rand16(ORC_FP16, rows, d + 11, 2.0);
    double *y = malloc((size_t)(rows * d) * sizeof(double));
    uint16_t *y16 = malloc((size_t)(rows * d) * 2);
    uint8_t *q = malloc((size_t)(rows * d));
    float *sc = malloc((size_t)rows * sizeof(float));
    EXPECT(orc_silu_and_mul(ORC_FP16, rows, d, gate, d + 5, up, d + 11, y, y16, mode, 0.02f, q, sc) == 0,
           "orc_silu_and_mul");
    free(gate); free(up); free(y); free(y16); free(q); free(sc);
  }
  EXPECT(fabs(orc_silu(0.0)) == 0.0, "silu(0)");

  /* GEMM: ragged K, padded strides, scale modes */
  const int64_t gshapes[][3] = {{1, 1, 16}, {3, 17, 48}, {5, 40, 300}, {2, 9, 1040}};
  for (int s = 0; s < 4; ++s) {
    const int64_t m = gshapes[s][0], n = gshapes[s][1], k = gshapes[s][2];
    const int64_t lda = k + 16 * (s & 1), ldb = k + 32 * (s & 1);
    uint8_t *a = rand_codes(m * lda), *b = rand_codes(n * ldb);
    float *sa = malloc((size_t)m * sizeof(float)), *sb = malloc((size_t)n * sizeof(float));
    for (int64_t i = 0; i < m; ++i) sa[i] = (float)(0.01 + uniform());
    for (int64_t j = 0; j < n; ++j) sb[j] = (float)(0.01 + uniform());
    double *c = malloc((size_t)(m * n) * sizeof(double));
    uint16_t *c16 = malloc((size_t)(m * n) * 2);
    for (int per = 0; per < 2; ++per) {
      EXPECT(orc_fp8_gemm(m, n, k, a, lda, sa, per, b, ldb, sb, per, s & 1, c, c16) == 0,
             "orc_fp8_gemm");
    }
    EXPECT(orc_fp8_gemm(m, n, k, a, k - 1, sa, 1, b, ldb, sb, 1, 0, c, c16) == -1,
           "lda < k refused");
    free(a); free(b); free(sa); free(sb); free(c); free(c16);
  }

  if (failures) {
    fprintf(stderr, "%d check(s) failed\n", failures);
    return 1;
  }
  puts("oracle driver: all calls clean");
  return 0;
}
