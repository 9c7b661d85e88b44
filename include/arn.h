/*
 * arn.h -- C ABI of the MI355X (gfx950) residual-add + RMSNorm library.
 *
 * One operator in four forms (plus SwiGLU and an e4m3 GEMM further below).
 * For every row i of a 16-bit activation matrix (bf16 or fp16), H = hidden:
 *
 *     r   = x[i] + residual[i]          (fused forms; plain forms use r = x[i])
 *     residual[i] <- r                   rounded to the 16-bit type
 *     y   = r / sqrt(mean_j(r_j^2) + eps) * w
 *     out[i] <- y                        16-bit, or OCP e4m3 codes (_fp8)
 *
 * RMSNorm is the definition of Zhang & Sennrich, "Root Mean Square Layer
 * Normalization" (NeurIPS 2019), eq. 4.  Fusing the residual add, the RMS
 * normalisation and the FP8 conversion into one pass over each row is the
 * first kernel of "Custom CUDA kernels juice Llama 3.1 405B on AMD MI300X,
 * skipping Nvidia lock-in" (paragraph 2).  The argument rules follow the
 * vLLM API page "vllm.kernels.aiter_ops" (attributes rms_add_no_var_16bit_only
 * and rms_no_var_16bit_only, and flatten_to_2d_is_free): 16-bit activations
 * only, a weight of the same dtype or none, and 2-D rows whose elements are
 * contiguous -- a layout that is not expressible that way is refused, never
 * copied, so the caller can fall back as vLLM's op priority list does.  The
 * four named entry points take the mean over all H channels, as those
 * wrappers require; arn_norm serves the same forms plus a variance-size
 * override.  Further below: the SwiGLU activation and the e4m3 GEMM that
 * consume and produce the same codes and scales.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Pointers are DEVICE pointers owned by the caller (hipMalloc, or a
 *    framework's allocator).  The library allocates nothing and keeps no
 *    state across calls other than a lazily filled, thread-safe per-device
 *    cache of the CU count.  (The test and tuning aids of arn_tuning.h keep
 *    per-thread settings that change only the calling thread's own calls.)
 *  - Layout: row-major, element stride 1, row stride given per tensor in
 *    ELEMENTS of that tensor (one e4m3 code = one element).  stride >= hidden.
 *    Elements [hidden, stride) of a row are neither read nor written.
 *  - dtype: ARN_BF16 or ARN_FP16, shared by x, residual, weight and 16-bit out.
 *  - weight: hidden elements of dtype, or NULL meaning w = 1.
 *  - eps: finite and >= 0, added to the mean square inside the square root.
 *  - Arithmetic: fp32 accumulation; the residual sum is one fp32 add rounded
 *    to nearest-even 16-bit; y is computed from that rounded sum.
 *  - Aliasing: out may equal x (same pointer and stride: in-place); residual
 *    must not overlap x or out; any other overlap is undefined.
 *  - Asynchrony: the call validates its arguments on the host, enqueues one
 *    kernel on `stream` and returns; execution errors surface at the
 *    caller's next synchronisation, as in HIP.  rows == 0 launches nothing.
 *  - Return value: ARN_OK, or
 *      ARN_EINVAL       an argument is invalid (nothing is launched);
 *      ARN_EUNSUPPORTED valid but not served, e.g. hidden above the largest
 *                       compiled row size (nothing is launched): rows up to
 *                       65536 elements when hidden and every row stride are
 *                       multiples of 4 and the 16-bit bases are 8-byte
 *                       aligned (e4m3 out: 4-byte), else 32768 when they are
 *                       multiples of 2 (4-byte / 2-byte aligned), else 16384;
 *      ARN_ELAUNCH      the HIP runtime refused the launch.
 *    No C++ exception crosses this interface.
 */
#ifndef ARN_H
#define ARN_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ARN_ABI_VERSION 6

enum arn_dtype { ARN_BF16 = 0, ARN_FP16 = 1 };
enum arn_fp8_mode { ARN_FP8_STATIC = 0, ARN_FP8_DYNAMIC = 1 };
enum arn_status { ARN_OK = 0, ARN_EINVAL = 1, ARN_EUNSUPPORTED = 2, ARN_ELAUNCH = 3 };

/*
 * Plain RMSNorm: out[i] = x[i] / sqrt(mean(x[i]^2) + eps) * w.
 * (vllm.kernels.aiter_ops, rms_no_var_16bit_only.)
 *   out, out_stride : rows x hidden of dtype, written.
 *   x, x_stride     : rows x hidden of dtype, read.
 */
int arn_rmsnorm(void *out, int64_t out_stride,
                const void *x, int64_t x_stride,
                const void *weight, float eps,
                int64_t rows, int64_t hidden, int dtype, hipStream_t stream);

/*
 * Fused residual add + RMSNorm.  residual[i] is read, replaced by the
 * rounded r = x[i] + residual[i], and out[i] = RMSNorm(r).
 * (vllm.kernels.aiter_ops, rms_add_no_var_16bit_only; the residual and
 * RMS-norm steps of the fused kernel in "Custom CUDA kernels juice Llama
 * 3.1 405B on AMD MI300X", paragraph 2.)
 *   residual, residual_stride : rows x hidden of dtype, read then written.
 */
int arn_fused_add_rmsnorm(void *out, int64_t out_stride,
                          const void *x, int64_t x_stride,
                          void *residual, int64_t residual_stride,
                          const void *weight, float eps,
                          int64_t rows, int64_t hidden, int dtype, hipStream_t stream);

/*
 * RMSNorm with an OCP e4m3 (E4M3FN) output, round to nearest even,
 * saturating at +-448.  The FP8 step of the fused kernel in "Custom CUDA
 * kernels juice Llama 3.1 405B on AMD MI300X" (paragraph 2).
 *   out, out_stride : rows x hidden bytes of e4m3 codes, written.
 *   scale           : fp8_mode ARN_FP8_STATIC -- ONE fp32 on the device, the
 *                     dequant scale s, read: code = e4m3(y / s), y ~ code * s.
 *                     s must be a positive normal fp32 number (2^-126 up to
 *                     the largest finite value); it is read by the kernel,
 *                     so it is not checked.
 *                     fp8_mode ARN_FP8_DYNAMIC -- `rows` fp32 on the device,
 *                     written: scale[i] = max_j |y_ij| / 448 rounded to fp32
 *                     and code = e4m3(y / scale[i]); a row whose max is 0
 *                     gets scale 0 and all-zero codes.  Rows whose max or
 *                     products leave fp32's range are served too: a scale
 *                     that rounds to a subnormal, to zero or past the
 *                     largest finite value is stored as rounded, and the
 *                     codes follow the stored value.
 *   Codes are within one e4m3 step of e4m3(y / scale) for exact y: the
 *   kernel forms the quotient in fp32, so a value within about one fp32
 *   rounding of a tie between two codes may take either.
 */
int arn_rmsnorm_fp8(uint8_t *out, int64_t out_stride, float *scale, int fp8_mode,
                    const void *x, int64_t x_stride,
                    const void *weight, float eps,
                    int64_t rows, int64_t hidden, int dtype, hipStream_t stream);

/* Fused residual add + RMSNorm + e4m3 output: the full single-pass kernel
 * of "Custom CUDA kernels juice Llama 3.1 405B on AMD MI300X" (paragraph 2).
 * Arguments as in arn_fused_add_rmsnorm and arn_rmsnorm_fp8. */
int arn_fused_add_rmsnorm_fp8(uint8_t *out, int64_t out_stride, float *scale, int fp8_mode,
                              const void *x, int64_t x_stride,
                              void *residual, int64_t residual_stride,
                              const void *weight, float eps,
                              int64_t rows, int64_t hidden, int dtype, hipStream_t stream);

/*
 * All four norm forms through one descriptor, plus a variance-size
 * override: the mean of squares runs over the first `variance_size`
 * channels only (1 <= variance_size <= hidden; 0 means hidden) and still
 * normalises every channel -- vLLM's RMSNorm variance_size_override, which
 * the AITER wrappers of "vllm.kernels.aiter_ops" (rms_add_no_var_16bit_only)
 * decline and this library serves.
 *   struct_size   : sizeof(arn_norm_args), checked (EINVAL if smaller)
 *   out_format    : ARN_OUT_16BIT, ARN_OUT_FP8_STATIC or ARN_OUT_FP8_DYNAMIC
 *   residual      : NULL selects plain RMSNorm, else the fused form
 *   scale         : as in arn_rmsnorm_fp8 (ignored for 16-bit output)
 * Other fields and the return value as in the entry points above.
 * With variance_size below hidden a channel outside the mean can be far
 * larger than the row's rms.  The 16-bit and bf16 static outputs form
 * (r_j * rsqrt(ms + eps)) * w_j in fp32 in that order, so an element whose
 * first product passes fp32's largest value (about 3.4e38) comes out
 * infinite (static: saturated) even where a weight below one would bring
 * y_j back into range.  At the full variance size that product stays below
 * sqrt(hidden).
 */
enum arn_out_format { ARN_OUT_16BIT = 0, ARN_OUT_FP8_STATIC = 1, ARN_OUT_FP8_DYNAMIC = 2 };

typedef struct arn_norm_args {
  size_t struct_size;
  int dtype;
  int out_format;
  void *out;
  int64_t out_stride;
  float *scale;
  const void *x;
  int64_t x_stride;
  void *residual;
  int64_t residual_stride;
  const void *weight;
  float eps;
  int64_t rows;
  int64_t hidden;
  int64_t variance_size;
  hipStream_t stream;
} arn_norm_args;

int arn_norm(const arn_norm_args *args);

/*
 * The reduction of an all-reduce fused with the residual add + RMSNorm: the
 * step that follows a tensor-parallel attention or MLP block, where each of
 * nparts ranks holds a partial sum of the same rows.  AITER supplies such
 * communication kernels and SGLang takes the all-reduce and the RMSNorm
 * together (page "AITER: AMD's operator library for ROCm ...", section
 * "Where it is actually used").  This is the kernel of one rank: for every
 * element the nparts partial values are added in fp32 in rank order (part 0
 * first) and rounded once to 16 bits -- what the all-reduce would return --
 * and that row then goes through the fused add + norm exactly as x does in
 * arn_norm.  Across GPUs the part pointers would be the peers' buffers,
 * mapped over xGMI; here any device pointers work.
 *   parts        : HOST array of nparts (1..8) device pointers, each rows x
 *                  hidden of dtype with row stride parts_stride elements.
 *   residual     : as in arn_norm (NULL: no residual add).
 *   out, scale, out_format, weight, eps, rows, hidden, stream : as in arn_norm
 *                  (no variance-size override).
 *   out may equal parts[0] (same stride); no other overlap.
 * Served rows: up to 32768 elements with 16-byte aligned rows (hidden and
 * strides multiples of 8), 16384 / 8192 / 4096 with 8 / 4 / 2-byte
 * alignment.  Returns as the other entry points.
 */
typedef struct arn_sum_norm_args {
  size_t struct_size;           /* sizeof(arn_sum_norm_args) */
  int dtype;
  int out_format;               /* ARN_OUT_16BIT, ARN_OUT_FP8_STATIC, ARN_OUT_FP8_DYNAMIC */
  void *out;
  int64_t out_stride;
  float *scale;
  const void *const *parts;
  int nparts;
  int64_t parts_stride;
  void *residual;
  int64_t residual_stride;
  const void *weight;
  float eps;
  int64_t rows;
  int64_t hidden;
  hipStream_t stream;
} arn_sum_norm_args;

int arn_sum_add_rmsnorm(const arn_sum_norm_args *args);

/*
 * SwiGLU activation: out[i][j] = silu(gate[i][j]) * up[i][j], j < d, with
 * silu(g) = g / (1 + exp(-g)) (Shazeer, "GLU Variants Improve Transformer",
 * 2020, FFN_SwiGLU with Swish_1).  The usual layout is one [rows, 2d] tensor
 * from the fused gate/up projection: gate = base, up = base + d, both with
 * that tensor's row stride; separate tensors work too.  All of gate, up and
 * out are of `dtype`; fp32 arithmetic, one rounding of the output (lanes
 * holding a gate at or below -80, where exp(-|g|) nears fp32's subnormal
 * range, and rows whose outputs leave fp32's range are formed in fp64, so
 * every finite input is served to the stated tolerance).  The
 * second kernel of "Custom CUDA kernels juice Llama 3.1 405B on AMD MI300X"
 * (paragraph 2) fuses this activation with the FP8 cast, which is
 * arn_silu_and_mul_fp8.  out may not alias gate or up.  Conventions as above
 * (device pointers, element strides >= d, asynchronous on `stream`).
 */
int arn_silu_and_mul(void *out, int64_t out_stride,
                     const void *gate, int64_t gate_stride,
                     const void *up, int64_t up_stride,
                     int64_t rows, int64_t d, int dtype, hipStream_t stream);

/* SwiGLU with an OCP e4m3 output; `scale` and fp8_mode as in
 * arn_rmsnorm_fp8 (static: one dequant scale read; dynamic: `rows` scales
 * max_j |y_ij| / 448 written).  The static kind forms y in fp32 before the
 * multiply by 1/s, so an output with |y| >= 2^128 saturates even where y/s
 * would not. */
int arn_silu_and_mul_fp8(uint8_t *out, int64_t out_stride, float *scale, int fp8_mode,
                         const void *gate, int64_t gate_stride,
                         const void *up, int64_t up_stride,
                         int64_t rows, int64_t d, int dtype, hipStream_t stream);

/*
 * e4m3 "skinny" GEMM for decode-sized activations (the third kernel of
 * "Custom CUDA kernels juice Llama 3.1 405B on AMD MI300X", paragraph 2):
 *     c[i][j] = sa(i) * sb(j) * sum_{t<k} dec(a[i][t]) * dec(b[j][t])
 * with OCP e4m3 codes: a is m x k activations (row stride lda BYTES), e.g.
 * the codes of arn_*_fp8; b is the n x k weight of a linear layer stored
 * out-feature major (row stride ldb bytes).  scale_a holds m per-row
 * dequant scales (a_per_row != 0) or one; scale_b holds n per-row scales
 * (b_per_row != 0) or one.  c is m x n of out_dtype (bf16/fp16, row stride
 * ldc elements), fp32 accumulation, one rounding.  Served: 1 <= m <= 64,
 * k % 16 == 0, lda and ldb multiples of 16, a and b 16-byte aligned (else
 * ARN_EUNSUPPORTED).  m or n == 0 launches nothing.  Device pointers,
 * asynchronous on `stream`.
 */
int arn_fp8_gemm(void *c, int64_t ldc, int out_dtype,
                 const uint8_t *a, int64_t lda, const float *scale_a, int a_per_row,
                 const uint8_t *b, int64_t ldb, const float *scale_b, int b_per_row,
                 int64_t m, int64_t n, int64_t k, hipStream_t stream);

/*
 * Pre-shuffled weights.  The fp8 multiply that vLLM hands to AITER (page
 * "vllm/rocm/use_aiter=1 slows Gemma 4 on an AMD MI300X", section "Why the
 * fp8 Multiplies Run Slower") reads its weight in a pre-shuffled layout.
 * Here the shuffled copy is a sequence of 2 KiB tiles, one per 16 weight
 * rows and 128-wide k step, each laid out so that every load instruction of
 * the GEMM reads 1 KiB contiguous bytes, and stored k-step major within
 * panels of at most 1 GiB (all column tiles of a panel for step 0, then for
 * step 1, ...), so that the GEMM's blocks read one compact region at a
 * time.  Rows past n and k past the last whole step are zero codes.  The
 * layout is private to this library: produce it with
 * arn_fp8_weight_preshuffle and read it only with arn_fp8_gemm_preshuffled.
 *
 * arn_fp8_weight_preshuffled_bytes: size of the copy for an n x k weight
 * (ceil(n/16) * ceil(k/128) * 2048), or -1 for n < 0 or k <= 0.
 *
 * arn_fp8_weight_preshuffle: writes the copy of the n x k row-major weight b
 * (row stride ldb >= k bytes, any alignment) into dst (caller-allocated, the
 * size above, 16-byte aligned, not overlapping b).  Served: k <= 2^23.
 * Asynchronous on `stream`; done once per weight.
 *
 * arn_fp8_gemm_preshuffled: arn_fp8_gemm with the weight given as that copy
 * (same n and k as at the shuffle); same results, same served shapes.
 */
int64_t arn_fp8_weight_preshuffled_bytes(int64_t n, int64_t k);
int arn_fp8_weight_preshuffle(uint8_t *dst, const uint8_t *b, int64_t ldb,
                              int64_t n, int64_t k, hipStream_t stream);
int arn_fp8_gemm_preshuffled(void *c, int64_t ldc, int out_dtype,
                             const uint8_t *a, int64_t lda, const float *scale_a,
                             int a_per_row, const uint8_t *b_shuffled,
                             const float *scale_b, int b_per_row,
                             int64_t m, int64_t n, int64_t k, hipStream_t stream);

/*
 * Split-K variants: with a workspace, K is also divided across several
 * blocks per output tile when that fills the GPU better (small N, or N not
 * a multiple of the CU count's worth of tiles); the block that completes a
 * tile last sums the partial tiles in a fixed order, so results are
 * deterministic for a given shape and device.
 *   arn_fp8_gemm_workspace_bytes: bytes the workspace needs for up to
 *     m x n outputs (about 8 x 64 x (n rounded up to 64) x 4 for m > 32,
 *     a half or a quarter of that for m <= 32 or 16), or -1 for m < 0,
 *     n < 0 or k <= 0.  A workspace sized for the largest shape serves
 *     every smaller one.
 *   workspace: device memory of at least that size, 256-byte aligned,
 *     ZERO-FILLED before its first use; every completed call leaves it
 *     ready for the next one, whatever the shape.  Calls that may run at
 *     the same time (other streams) need separate workspaces.  NULL means
 *     no split (as the plain entry points).
 * Other arguments and results as in arn_fp8_gemm / arn_fp8_gemm_preshuffled.
 */
int64_t arn_fp8_gemm_workspace_bytes(int64_t m, int64_t n, int64_t k);
int arn_fp8_gemm_ws(void *c, int64_t ldc, int out_dtype,
                    const uint8_t *a, int64_t lda, const float *scale_a, int a_per_row,
                    const uint8_t *b, int64_t ldb, const float *scale_b, int b_per_row,
                    int64_t m, int64_t n, int64_t k, void *workspace, size_t workspace_bytes,
                    hipStream_t stream);
int arn_fp8_gemm_preshuffled_ws(void *c, int64_t ldc, int out_dtype,
                                const uint8_t *a, int64_t lda, const float *scale_a,
                                int a_per_row, const uint8_t *b_shuffled,
                                const float *scale_b, int b_per_row,
                                int64_t m, int64_t n, int64_t k, void *workspace,
                                size_t workspace_bytes, hipStream_t stream);

/*
 * arn_fp8_gemm_preshuffled_ws without a workspace argument, for callers
 * that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): the split-K partial
 * tiles and tile counters live in a device array inside the library, of
 * ARN_NOALLOC_SCRATCH_BYTES (8 MiB) per GPU, held until the process ends.
 * The call allocates nothing and calls no allocating routine.
 *   - Served: shapes whose workspace (arn_fp8_gemm_workspace_bytes) fits
 *     the array -- m <= 64 with n <= 4032, m <= 32 with n <= 8128, m <= 16
 *     with n <= 16256 -- else ARN_EUNSUPPORTED, nothing launched (use
 *     arn_fp8_gemm_preshuffled_ws with a workspace of your own).
 *   - The array is shared by every call on one GPU: calls that may run at
 *     the same time on that GPU (other streams, other threads) race and
 *     give wrong results; serialise them.  Each completed call leaves the
 *     array ready for the next one.  The first call on a device clears the
 *     array's counters with a small kernel on `stream`.
 *   - Other arguments, results and status codes as in
 *     arn_fp8_gemm_preshuffled_ws (bit-identical results for the same
 *     shape and device); ARN_ELAUNCH if the array cannot be located.
 */
#define ARN_NOALLOC_SCRATCH_BYTES (8u << 20)
int arn_fp8_gemm_preshuffled_noalloc(void *c, int64_t ldc, int out_dtype,
                                     const uint8_t *a, int64_t lda, const float *scale_a,
                                     int a_per_row, const uint8_t *b_shuffled,
                                     const float *scale_b, int b_per_row,
                                     int64_t m, int64_t n, int64_t k, hipStream_t stream);

/* Static, NUL-terminated description of a status code. */
const char *arn_status_str(int status);

/* ARN_ABI_VERSION of the loaded library. */
int arn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ARN_H */
