/*
 * oracle.c -- plain, slow, obviously correct CPU reference (fp64).
 *
 * TEST INFRASTRUCTURE ONLY: called by the test suite, the smoke check and
 * the CPU-baseline leg of the benchmark, never by the product path.  It
 * shares no code with the HIP library and includes none of its headers.
 *
 * What is computed, with the passages it follows:
 *   - RMSNorm itself is the textbook definition (Zhang & Sennrich, "Root
 *     Mean Square Layer Normalization", NeurIPS 2019, eq. 4):
 *         y_j = r_j / sqrt(mean_k(r_k^2) + eps) * w_j .
 *   - "Custom CUDA kernels juice Llama 3.1 405B on AMD MI300X, skipping
 *     Nvidia lock-in", paragraph 2: the first kernel fuses the residual
 *     connection, the RMS normalisation and the FP8 conversion.  So each
 *     row is r = x + residual (written back to the residual stream), then
 *     RMSNorm of r, then optionally an FP8 cast of y.
 *   - vLLM API docs "vllm.kernels.aiter_ops", attributes
 *     rms_add_no_var_16bit_only / rms_no_var_16bit_only: 16-bit (fp16 or
 *     bf16) activations, weight of the same dtype or None, and no
 *     variance-size override -- so the mean runs over all `hidden`
 *     channels, and a missing weight means w = 1.
 *   - The second kernel of that article fuses the SwiGLU activation with
 *     the FP8 cast.  SwiGLU is Shazeer, "GLU Variants Improve
 *     Transformer" (2020): Swish_1(x W) * (x V), Swish_1 = SiLU; here the
 *     two projections arrive as the gate and up halves of one row.
 *   - The third kernel of that article is a "skinny" GEMM for the small
 *     batch shapes of decoding; here it is the plain definition of a
 *     matrix product of decoded e4m3 codes times their dequant scales.
 *   - The FP8 format is OCP E4M3FN (bias 7, 3 mantissa bits, max 448, no
 *     infinities, NaN = S.1111.111).  "MI210 LLM Stack", key insight 4,
 *     counts 254 non-NaN e4m3 byte patterns, which is that format.
 *
 * Readings where the pages are silent (each one is a choice, listed with
 * its reason in the design notes of the repository):
 *   - y is computed from the rounded, stored residual r16, in fp64, and
 *     rounded once at the end.
 *   - eps is an fp32 value widened exactly and added inside the sqrt.
 *   - Static FP8: the caller passes the dequant scale s; q = E(y / s).
 *   - Dynamic FP8: amax = max_j |y_j|, scale = fp32(amax / 448) stored,
 *     q = E(y / scale); a row with amax == 0 gets scale 0 and zero codes.
 *   - The e4m3 code is chosen from the quotient y / s as fp64 computes it,
 *     with no narrower rounding in between: E rounds that value itself.
 */
#include "oracle.h"

#include <math.h>
#include <stddef.h>
#include <stdlib.h>

/* --------------------------------------------------------------------- */
/* IEEE-style binary formats (IEEE 754-2008 section 3.4 for binary16;    */
/* bfloat16 is binary32 with the low 16 mantissa bits removed).          */
/* --------------------------------------------------------------------- */

typedef struct {
    int exp_bits;  /* width of the exponent field        */
    int man_bits;  /* width of the stored mantissa field */
    int bias;      /* exponent bias                      */
} orc_format;

static orc_format format_of(int dtype)
{
    orc_format f;
    if (dtype == ORC_BF16) {
        f.exp_bits = 8;
        f.man_bits = 7;
        f.bias = 127;
    } else {
        f.exp_bits = 5;
        f.man_bits = 10;
        f.bias = 15;
    }
    return f;
}

/* value = (-1)^s * 2^(e - bias) * (1 + m / 2^M) for 0 < e < all-ones,
 *         (-1)^s * 2^(1 - bias) * (m / 2^M)     for e == 0,
 *         +-Inf / NaN                            for e == all-ones. */
double orc_decode16(int dtype, uint16_t bits)
{
    orc_format f = format_of(dtype);
    int sign = (bits >> 15) & 1;
    int emax_field = (1 << f.exp_bits) - 1;
    int e = (bits >> f.man_bits) & emax_field;
    int m = bits & ((1 << f.man_bits) - 1);
    double mag;

    if (e == emax_field) {
        mag = (m == 0) ? INFINITY : NAN;
    } else if (e == 0) {
        mag = ldexp((double)m, 1 - f.bias - f.man_bits);
    } else {
        mag = ldexp((double)((1 << f.man_bits) + m), e - f.bias - f.man_bits);
    }
    return sign ? -mag : mag;
}

/* Round a non-negative integer-valued-or-not double n to an integer,
 * halfway cases to the even neighbour. */
static double round_half_even(double n)
{
    double lo = floor(n);
    double frac = n - lo; /* exact: n < 2^53 in every caller */
    if (frac > 0.5) {
        return lo + 1.0;
    }
    if (frac == 0.5 && fmod(lo, 2.0) != 0.0) {
        return lo + 1.0;
    }
    return lo;
}

/* Exponent e with 2^e <= a < 2^(e+1), for finite a > 0. */
static int floor_log2(double a)
{
    int k;
    (void)frexp(a, &k); /* a = f * 2^k, 0.5 <= f < 1 */
    return k - 1;
}

uint16_t orc_encode16(int dtype, double v)
{
    orc_format f = format_of(dtype);
    int emax_field = (1 << f.exp_bits) - 1;
    uint16_t sign = signbit(v) ? (uint16_t)0x8000 : (uint16_t)0;
    uint16_t inf_bits = (uint16_t)(emax_field << f.man_bits);
    double a = fabs(v);
    int emin = 1 - f.bias;
    int e;
    double quantum, n;

    if (isnan(v)) {
        return (uint16_t)(sign | inf_bits | (1 << (f.man_bits - 1)));
    }
    if (isinf(v)) {
        return (uint16_t)(sign | inf_bits);
    }
    if (a == 0.0) {
        return sign;
    }

    e = floor_log2(a);
    if (e < emin) {
        e = emin; /* subnormal range: fixed quantum 2^(emin - M) */
    }
    quantum = ldexp(1.0, e - f.man_bits);
    n = round_half_even(a / quantum); /* the division is a power-of-2 scaling */

    if (n == ldexp(1.0, f.man_bits + 1)) { /* rounded up to the next binade */
        n = ldexp(1.0, f.man_bits);
        e += 1;
    }
    if (n < ldexp(1.0, f.man_bits)) { /* subnormal (only possible at e == emin) */
        return (uint16_t)(sign | (uint16_t)n);
    }
    if (e + f.bias >= emax_field) { /* overflow */
        return (uint16_t)(sign | inf_bits);
    }
    return (uint16_t)(sign | (uint16_t)((e + f.bias) << f.man_bits) |
                      (uint16_t)(n - ldexp(1.0, f.man_bits)));
}

/* --------------------------------------------------------------------- */
/* OCP 8-bit floating point, E4M3FN ("OCP 8-bit Floating Point           */
/* Specification (OFP8)", rev. 1.0, table 1): bias 7, exponent field     */
/* 0..15, S.1111.111 is NaN, no infinities, max normal 1.75 * 2^8 = 448, */
/* subnormals m * 2^-9.                                                  */
/* --------------------------------------------------------------------- */

double orc_e4m3_decode(uint8_t code)
{
    int sign = (code >> 7) & 1;
    int e = (code >> 3) & 0xF;
    int m = code & 0x7;
    double mag;

    if (e == 15 && m == 7) {
        mag = NAN;
    } else if (e == 0) {
        mag = ldexp((double)m, -9);
    } else {
        mag = ldexp((double)(8 + m), e - 7 - 3);
    }
    return sign ? -mag : mag;
}

uint8_t orc_e4m3_encode(double v)
{
    uint8_t sign = signbit(v) ? (uint8_t)0x80 : (uint8_t)0;
    double a = fabs(v);
    int e;
    double n;

    if (isnan(v)) {
        return 0x7F;
    }
    if (a >= 448.0) { /* saturate, Inf included */
        return (uint8_t)(sign | 0x7E);
    }
    if (a == 0.0) {
        return sign;
    }

    e = floor_log2(a);
    if (e < -6) {
        e = -6; /* subnormal range: quantum 2^-9 */
    }
    n = round_half_even(ldexp(a, 3 - e)); /* a / 2^(e-3) */
    if (n == 16.0) {
        n = 8.0;
        e += 1;
    }
    if (n < 8.0) { /* subnormal, or zero after rounding */
        return (uint8_t)(sign | (uint8_t)n);
    }
    /* a < 448 keeps the result at or below 448 = (e 8, n 14). */
    return (uint8_t)(sign | (uint8_t)((e + 7) << 3) | (uint8_t)(n - 8.0));
}

/* --------------------------------------------------------------------- */
/* The operator, one row at a time.                                      */
/* --------------------------------------------------------------------- */

/* Step 1 (residual connection): r_j = x_j + res_j, exact sum rounded once
 * to double and then to the storage type; the rounded value is what the
 * residual stream keeps and what the rest of the row is computed from. */
static void residual_add_row(int dtype, int64_t hidden, const uint16_t *x,
                             const uint16_t *res, uint16_t *r16, double *r)
{
    int64_t j;
    for (j = 0; j < hidden; j++) {
        double sum = orc_decode16(dtype, x[j]) + orc_decode16(dtype, res[j]);
        r16[j] = orc_encode16(dtype, sum);
        r[j] = orc_decode16(dtype, r16[j]);
    }
}

/* The residual step alone, for n independent pairs: out[i] is the stored
 * residual for x[i] + res[i], exactly as a row computes it. */
int orc_residual16(int dtype, int64_t n, const uint16_t *x, const uint16_t *res,
                   uint16_t *out)
{
    double r[1024];
    int64_t i;
    if (dtype != ORC_BF16 && dtype != ORC_FP16) {
        return 1;
    }
    if (n < 0 || (n > 0 && (x == NULL || res == NULL || out == NULL))) {
        return 1;
    }
    for (i = 0; i < n; i += 1024) {
        int64_t len = n - i < 1024 ? n - i : 1024;
        residual_add_row(dtype, len, x + i, res + i, out + i, r);
    }
    return 0;
}

/* All-reduce reduction step, per element: fp32 accumulation in rank order,
 * then one rounding to the storage type.  (float) of a decoded 16-bit value
 * is exact; each float addition is one IEEE single-precision add (the file
 * is compiled without contraction or fast-math). */
int orc_sum_parts16(int dtype, int nparts, const uint16_t *const *parts, int64_t parts_stride,
                    int64_t rows, int64_t hidden, uint16_t *x16_out)
{
    int64_t i, j;
    int g;
    if ((dtype != ORC_BF16 && dtype != ORC_FP16) || nparts < 1 || parts == NULL ||
        rows < 0 || hidden <= 0 || parts_stride < hidden || x16_out == NULL) {
        return -1;
    }
    for (g = 0; g < nparts; g++) {
        if (parts[g] == NULL) {
            return -1;
        }
    }
    for (i = 0; i < rows; i++) {
        for (j = 0; j < hidden; j++) {
            float total = (float)orc_decode16(dtype, parts[0][i * parts_stride + j]);
            for (g = 1; g < nparts; g++) {
                total = total + (float)orc_decode16(dtype, parts[g][i * parts_stride + j]);
            }
            x16_out[i * hidden + j] = orc_encode16(dtype, (double)total);
        }
    }
    return 0;
}

/* Plain RMSNorm has no residual: r is x itself. */
static void copy_row(int dtype, int64_t hidden, const uint16_t *x, uint16_t *r16,
                     double *r)
{
    int64_t j;
    for (j = 0; j < hidden; j++) {
        r16[j] = x[j];
        r[j] = orc_decode16(dtype, x[j]);
    }
}

/* Step 2: mean of squares over the first n channels, summed left to right.
 * n = hidden, unless the caller overrides the variance size (vLLM's RMSNorm
 * variance_size_override: the variance of the first n channels normalises
 * all of them). */
static double mean_square(int64_t n, const double *r)
{
    double sum = 0.0;
    int64_t j;
    for (j = 0; j < n; j++) {
        sum += r[j] * r[j];
    }
    return sum / (double)n;
}

/* Step 3: y_j = r_j * (1 / sqrt(ms + eps)) * w_j. */
static void normalise_row(int dtype, int64_t hidden, const double *r, double ms,
                          float eps, const uint16_t *weight, double *y)
{
    double inv = 1.0 / sqrt(ms + (double)eps);
    int64_t j;
    for (j = 0; j < hidden; j++) {
        double w = weight ? orc_decode16(dtype, weight[j]) : 1.0;
        y[j] = r[j] * inv * w;
    }
}

/* Step 4s: static per-tensor FP8, q_j = E(y_j / s). */
static void quant_static_row(int64_t hidden, const double *y, float s, uint8_t *q)
{
    int64_t j;
    for (j = 0; j < hidden; j++) {
        q[j] = orc_e4m3_encode(y[j] / (double)s);
    }
}

/* Step 4d: dynamic per-row FP8.  amax = max |y_j| (NaN if any y_j is NaN),
 * scale = fp32(amax / 448), q_j = E(y_j / scale); amax == 0 gives scale 0
 * and all-zero codes. */
static float quant_dynamic_row(int64_t hidden, const double *y, uint8_t *q)
{
    double amax = 0.0;
    float scale;
    int64_t j;

    for (j = 0; j < hidden; j++) {
        if (isnan(y[j])) {
            amax = NAN;
            break;
        }
        if (fabs(y[j]) > amax) {
            amax = fabs(y[j]);
        }
    }
    scale = (float)(amax / 448.0);
    for (j = 0; j < hidden; j++) {
        if (amax == 0.0) {
            q[j] = 0x00;
        } else {
            q[j] = orc_e4m3_encode(y[j] / (double)scale);
        }
    }
    return scale;
}

int orc_add_rmsnorm(int dtype, int64_t rows, int64_t hidden,
                    const uint16_t *x, int64_t x_stride,
                    const uint16_t *residual, int64_t residual_stride,
                    const uint16_t *weight, float eps,
                    uint16_t *r16_out, double *y_out, uint16_t *y16_out,
                    int fp8_mode, float static_scale,
                    uint8_t *q_out, float *scale_out)
{
    return orc_add_rmsnorm_var(dtype, rows, hidden, hidden, x, x_stride, residual,
                               residual_stride, weight, eps, r16_out, y_out, y16_out,
                               fp8_mode, static_scale, q_out, scale_out);
}

int orc_add_rmsnorm_var(int dtype, int64_t rows, int64_t hidden, int64_t variance_size,
                        const uint16_t *x, int64_t x_stride,
                        const uint16_t *residual, int64_t residual_stride,
                        const uint16_t *weight, float eps,
                        uint16_t *r16_out, double *y_out, uint16_t *y16_out,
                        int fp8_mode, float static_scale,
                        uint8_t *q_out, float *scale_out)
{
    uint16_t *r16;
    double *r, *y;
    uint8_t *q;
    int64_t i, j;

    if ((dtype != ORC_BF16 && dtype != ORC_FP16) || rows < 0 || hidden <= 0 ||
        variance_size <= 0 || variance_size > hidden ||
        x == NULL || x_stride < hidden ||
        (residual != NULL && residual_stride < hidden) ||
        (fp8_mode != ORC_FP8_NONE && fp8_mode != ORC_FP8_STATIC &&
         fp8_mode != ORC_FP8_DYNAMIC)) {
        return -1;
    }

    r16 = (uint16_t *)malloc((size_t)hidden * sizeof(uint16_t));
    r = (double *)malloc((size_t)hidden * sizeof(double));
    y = (double *)malloc((size_t)hidden * sizeof(double));
    q = (uint8_t *)malloc((size_t)hidden);
    if (!r16 || !r || !y || !q) {
        free(r16);
        free(r);
        free(y);
        free(q);
        return -1;
    }

    for (i = 0; i < rows; i++) {
        const uint16_t *xi = x + i * x_stride;
        double ms;
        float scale = 0.0f;

        if (residual != NULL) {
            residual_add_row(dtype, hidden, xi, residual + i * residual_stride, r16, r);
        } else {
            copy_row(dtype, hidden, xi, r16, r);
        }
        ms = mean_square(variance_size, r);
        normalise_row(dtype, hidden, r, ms, eps, weight, y);

        if (fp8_mode == ORC_FP8_STATIC) {
            quant_static_row(hidden, y, static_scale, q);
        } else if (fp8_mode == ORC_FP8_DYNAMIC) {
            scale = quant_dynamic_row(hidden, y, q);
        }

        for (j = 0; j < hidden; j++) {
            if (r16_out) {
                r16_out[i * hidden + j] = r16[j];
            }
            if (y_out) {
                y_out[i * hidden + j] = y[j];
            }
            if (y16_out) {
                y16_out[i * hidden + j] = orc_encode16(dtype, y[j]);
            }
            if (q_out && fp8_mode != ORC_FP8_NONE) {
                q_out[i * hidden + j] = q[j];
            }
        }
        if (scale_out && fp8_mode == ORC_FP8_DYNAMIC) {
            scale_out[i] = scale;
        }
    }

    free(r16);
    free(r);
    free(y);
    free(q);
    return 0;
}

/* --------------------------------------------------------------------- */
/* SwiGLU: y = silu(gate) * up.                                          */
/* --------------------------------------------------------------------- */

/* silu(g) = g * sigmoid(g) with sigmoid(g) = 1 / (1 + exp(-g)).  For
   g < 0 sigmoid is taken in the equal form exp(g) / (1 + exp(g)): exp(-g)
   overflows fp64 below about -709.8 while sigmoid(g) is still
   representable down to about -745. */
double orc_silu(double g)
{
    if (g < 0.0) {
        const double e = exp(g);
        return g * e / (1.0 + e);
    }
    return g / (1.0 + exp(-g));
}

int orc_silu_and_mul(int dtype, int64_t rows, int64_t d,
                     const uint16_t *gate, int64_t gate_stride,
                     const uint16_t *up, int64_t up_stride,
                     double *y_out, uint16_t *y16_out,
                     int fp8_mode, float static_scale,
                     uint8_t *q_out, float *scale_out)
{
    double *y;
    uint8_t *q;
    int64_t i, j;

    if ((dtype != ORC_BF16 && dtype != ORC_FP16) || rows < 0 || d <= 0 ||
        gate == NULL || up == NULL || gate_stride < d || up_stride < d ||
        (fp8_mode != ORC_FP8_NONE && fp8_mode != ORC_FP8_STATIC &&
         fp8_mode != ORC_FP8_DYNAMIC)) {
        return -1;
    }
    y = (double *)malloc((size_t)d * sizeof(double));
    q = (uint8_t *)malloc((size_t)d);
    if (!y || !q) {
        free(y);
        free(q);
        return -1;
    }

    for (i = 0; i < rows; i++) {
        float scale = 0.0f;
        for (j = 0; j < d; j++) {
            double g = orc_decode16(dtype, gate[i * gate_stride + j]);
            double u = orc_decode16(dtype, up[i * up_stride + j]);
            y[j] = orc_silu(g) * u;
        }
        if (fp8_mode == ORC_FP8_STATIC) {
            quant_static_row(d, y, static_scale, q);
        } else if (fp8_mode == ORC_FP8_DYNAMIC) {
            scale = quant_dynamic_row(d, y, q);
        }
        for (j = 0; j < d; j++) {
            if (y_out) {
                y_out[i * d + j] = y[j];
            }
            if (y16_out) {
                y16_out[i * d + j] = orc_encode16(dtype, y[j]);
            }
            if (q_out && fp8_mode != ORC_FP8_NONE) {
                q_out[i * d + j] = q[j];
            }
        }
        if (scale_out && fp8_mode == ORC_FP8_DYNAMIC) {
            scale_out[i] = scale;
        }
    }
    free(y);
    free(q);
    return 0;
}

/* --------------------------------------------------------------------- */
/* e4m3 GEMM: C = diag(sa) (dec(A) dec(B)^T) diag(sb).                    */
/* --------------------------------------------------------------------- */

int orc_fp8_gemm(int64_t m, int64_t n, int64_t k,
                 const uint8_t *a, int64_t lda, const float *sa, int a_per_row,
                 const uint8_t *b, int64_t ldb, const float *sb, int b_per_row,
                 int out_dtype, double *c_out, uint16_t *c16_out)
{
    int64_t i, j, t;

    if (m < 0 || n < 0 || k <= 0 || a == NULL || b == NULL || sa == NULL || sb == NULL ||
        lda < k || ldb < k || (out_dtype != ORC_BF16 && out_dtype != ORC_FP16)) {
        return -1;
    }
    for (i = 0; i < m; i++) {
        double scale_a = (double)(a_per_row ? sa[i] : sa[0]);
        for (j = 0; j < n; j++) {
            double scale_b = (double)(b_per_row ? sb[j] : sb[0]);
            double sum = 0.0;
            for (t = 0; t < k; t++) {
                double p = orc_e4m3_decode(a[i * lda + t]) * orc_e4m3_decode(b[j * ldb + t]);
                sum += p;
            }
            if (c_out) {
                c_out[i * n + j] = scale_a * scale_b * sum;
            }
            if (c16_out) {
                c16_out[i * n + j] = orc_encode16(out_dtype, scale_a * scale_b * sum);
            }
        }
    }
    return 0;
}
