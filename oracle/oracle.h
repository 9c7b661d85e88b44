/*
 * oracle.h -- plain fp64 CPU reference for residual-add + RMSNorm (+ OCP e4m3).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may include, link,
 * load or call this code: only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark do.  It shares no code, header, table or
 * constant with the HIP library.
 *
 * Every function computes the textbook definition, one step at a time, in
 * double precision; see oracle.c for the citation of each step.
 */
#ifndef ARN_ORACLE_H
#define ARN_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* 16-bit storage formats understood by the oracle. */
#define ORC_BF16 0
#define ORC_FP16 1

/* FP8 modes: none, per-tensor static scale, per-row dynamic scale. */
#define ORC_FP8_NONE    (-1)
#define ORC_FP8_STATIC  0
#define ORC_FP8_DYNAMIC 1

/* Exact decode of a 16-bit pattern (bf16 or IEEE binary16) to double. */
double orc_decode16(int dtype, uint16_t bits);

/* Round a double to the nearest 16-bit value, ties to even mantissa,
 * overflow to +-Inf, NaN to a quiet NaN. */
uint16_t orc_encode16(int dtype, double v);

/* Exact decode of an OCP E4M3FN code (0x7F / 0xFF decode to NaN). */
double orc_e4m3_decode(uint8_t code);

/* OCP E4M3FN encoder: nearest finite value, ties to even mantissa,
 * saturating at +-448, NaN -> 0x7F, signed zero kept. */
uint8_t orc_e4m3_encode(double v);

/* The stored residual of n independent pairs: out[i] = the 16-bit rounding
 * of x[i] + res[i] (the first step of a fused row).  Returns 0, or 1 for an
 * invalid argument. */
int orc_residual16(int dtype, int64_t n, const uint16_t *x, const uint16_t *res,
                   uint16_t *out);

/*
 * The operator, row by row.
 *   x, residual : rows x hidden 16-bit patterns, row strides in elements.
 *                 residual == NULL selects plain RMSNorm (r = x).
 *   weight      : hidden 16-bit patterns, or NULL for w = 1.
 *   eps         : fp32 value, widened exactly.
 * Outputs (each may be NULL; all dense, row stride = hidden):
 *   r16_out   : the rounded sum that is stored back into residual.
 *   y_out     : unrounded y in double.
 *   y16_out   : y rounded to the 16-bit type.
 *   q_out     : e4m3 codes (fp8_mode STATIC or DYNAMIC).
 *   scale_out : per-row dequant scales (DYNAMIC only, rows floats).
 * static_scale is the dequant scale s of STATIC mode (q = E(y / s)).
 * Returns 0, or -1 on an argument error.
 */
int orc_add_rmsnorm(int dtype, int64_t rows, int64_t hidden,
                    const uint16_t *x, int64_t x_stride,
                    const uint16_t *residual, int64_t residual_stride,
                    const uint16_t *weight, float eps,
                    uint16_t *r16_out, double *y_out, uint16_t *y16_out,
                    int fp8_mode, float static_scale,
                    uint8_t *q_out, float *scale_out);

/* The same with the mean of squares taken over the first variance_size
 * channels only (1 <= variance_size <= hidden); every channel is still
 * normalised by it. */
int orc_add_rmsnorm_var(int dtype, int64_t rows, int64_t hidden, int64_t variance_size,
                        const uint16_t *x, int64_t x_stride,
                        const uint16_t *residual, int64_t residual_stride,
                        const uint16_t *weight, float eps,
                        uint16_t *r16_out, double *y_out, uint16_t *y16_out,
                        int fp8_mode, float static_scale,
                        uint8_t *q_out, float *scale_out);

/*
 * The reduction of an all-reduce over nparts ranks, as one rank's kernel
 * would compute it before a fused residual add + RMSNorm: for each element,
 * the nparts 16-bit partial values are accumulated in fp32 in rank order
 * (part 0 first), and the fp32 total is rounded once to the 16-bit type:
 *     x16[i][j] = RNE16( fp32( ... fp32(fp32(p0) + p1) ... + p_{n-1} ) )
 * parts[g] points at rows x hidden patterns with row stride parts_stride.
 * x16_out is dense (row stride hidden).  Feeding x16_out as x to
 * orc_add_rmsnorm gives the fused all-reduce + add + norm.  Returns 0, or
 * -1 on an argument error.
 */
int orc_sum_parts16(int dtype, int nparts, const uint16_t *const *parts, int64_t parts_stride,
                    int64_t rows, int64_t hidden, uint16_t *x16_out);

/*
 * SwiGLU activation of a gate/up pair (Shazeer, "GLU Variants Improve
 * Transformer", 2020, the FFN_SwiGLU definition with Swish_1 = SiLU):
 *     y_j = silu(g_j) * u_j,   silu(g) = g / (1 + exp(-g)).
 * Row i reads gate[i*gate_stride + j] and up[i*up_stride + j], j < d (the
 * usual layout passes up = gate + d inside one [rows, 2d] tensor).
 * Outputs as in orc_add_rmsnorm (dense, row stride d; each may be NULL).
 */
double orc_silu(double g);
int orc_silu_and_mul(int dtype, int64_t rows, int64_t d,
                     const uint16_t *gate, int64_t gate_stride,
                     const uint16_t *up, int64_t up_stride,
                     double *y_out, uint16_t *y16_out,
                     int fp8_mode, float static_scale,
                     uint8_t *q_out, float *scale_out);

/*
 * e4m3 GEMM with dequant scales (the "skinny GEMM" that consumes the FP8
 * codes and per-row scales of the kernels above):
 *     C[m][n] = sa(m) * sb(n) * sum_k dec(A[m][k]) * dec(B[n][k])
 * A: M x K codes (row stride lda), B: N x K codes (row stride ldb, the
 * weight of a linear layer stored out-feature major), sa: M per-row scales
 * or 1 per-tensor scale (a_per_row = 0), sb likewise over N.  The sum runs
 * k = 0..K-1 in fp64.  Outputs (dense, row stride N; may be NULL): c_out in
 * fp64 and c16_out rounded to the 16-bit dtype.
 */
int orc_fp8_gemm(int64_t m, int64_t n, int64_t k,
                 const uint8_t *a, int64_t lda, const float *sa, int a_per_row,
                 const uint8_t *b, int64_t ldb, const float *sb, int b_per_row,
                 int out_dtype, double *c_out, uint16_t *c16_out);

#ifdef __cplusplus
}
#endif

#endif /* ARN_ORACLE_H */
