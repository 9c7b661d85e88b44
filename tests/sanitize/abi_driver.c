/*
 * abi_driver.c -- drives the host side of libarn's C ABI (argument checks,
 * status strings, size queries, tuning knobs, the plan buffer, the plan
 * query) along the paths that return before any HIP call: refused
 * arguments, empty calls and plan queries.
 * tests/sanitize/build.py links it with the library's objects, the host
 * code of arn_api.hip built under AddressSanitizer and
 * UndefinedBehaviorSanitizer, so an out-of-bounds access or undefined
 * operation in that code is reported.  No GPU is needed; device pointers
 * are stand-ins that are never dereferenced.  Exit status 0 on success.
 */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "arn.h"
#include "arn_tuning.h"

static int failures = 0;
#define EXPECT_EQ(got, want, what)                                                  \
  do {                                                                              \
    long long g_ = (long long)(got), w_ = (long long)(want);                        \
    if (g_ != w_) {                                                                 \
      fprintf(stderr, "FAILED: %s: got %lld, want %lld (line %d)\n", what, g_, w_, \
              __LINE__);                                                            \
      ++failures;                                                                   \
    }                                                                               \
  } while (0)

int main(void) {
  void *dev = (void *)(uintptr_t)0x100000;  /* 256-byte aligned stand-in, never read */
  uint8_t *dev8 = (uint8_t *)dev;
  float *devf = (float *)dev;
  const float nan = __builtin_nanf("");

  EXPECT_EQ(arn_abi_version(), ARN_ABI_VERSION, "abi version");
  for (int s = -2; s <= 5; ++s) {
    const char *m = arn_status_str(s);
    EXPECT_EQ(m != NULL && strlen(m) > 0, 1, "status string");
  }

  /* plain and fused norm: refusals, then an empty call */
  EXPECT_EQ(arn_rmsnorm(NULL, 64, dev, 64, dev, 1e-6f, 4, 64, ARN_BF16, 0), ARN_EINVAL, "null out");
  EXPECT_EQ(arn_rmsnorm(dev, 64, NULL, 64, dev, 1e-6f, 4, 64, ARN_BF16, 0), ARN_EINVAL, "null x");
  EXPECT_EQ(arn_rmsnorm(dev, 64, dev, 32, dev, 1e-6f, 4, 64, ARN_BF16, 0), ARN_EINVAL, "x stride");
  EXPECT_EQ(arn_rmsnorm(dev, 32, dev, 64, dev, 1e-6f, 4, 64, ARN_BF16, 0), ARN_EINVAL, "out stride");
  EXPECT_EQ(arn_rmsnorm(dev, 64, dev, 64, dev, 1e-6f, -1, 64, ARN_BF16, 0), ARN_EINVAL, "rows < 0");
  EXPECT_EQ(arn_rmsnorm(dev, 64, dev, 64, dev, 1e-6f, 4, 0, ARN_BF16, 0), ARN_EINVAL, "hidden 0");
  EXPECT_EQ(arn_rmsnorm(dev, 64, dev, 64, dev, 1e-6f, 4, 64, 7, 0), ARN_EINVAL, "dtype");
  EXPECT_EQ(arn_rmsnorm(dev, 64, dev, 64, dev, -1.0f, 4, 64, ARN_BF16, 0), ARN_EINVAL, "eps < 0");
  EXPECT_EQ(arn_rmsnorm(dev, 64, dev, 64, dev, nan, 4, 64, ARN_BF16, 0), ARN_EINVAL, "eps NaN");
  EXPECT_EQ(arn_rmsnorm(dev, 64, dev, 64, dev, 1e-6f, 0, 64, ARN_BF16, 0), ARN_OK, "no rows");
  EXPECT_EQ(arn_fused_add_rmsnorm(dev, 64, dev, 64, NULL, 64, dev, 1e-6f, 4, 64, ARN_FP16, 0),
            ARN_EINVAL, "null residual");
  EXPECT_EQ(arn_fused_add_rmsnorm(dev, 64, dev, 64, dev, 63, dev, 1e-6f, 4, 64, ARN_FP16, 0),
            ARN_EINVAL, "residual stride");
  EXPECT_EQ(arn_fused_add_rmsnorm(dev, 64, dev, 64, dev, 64, NULL, 1e-6f, 0, 64, ARN_FP16, 0),
            ARN_OK, "no rows, no weight");
  EXPECT_EQ(arn_rmsnorm_fp8(dev8, 64, NULL, ARN_FP8_STATIC, dev, 64, dev, 1e-6f, 4, 64, ARN_BF16, 0),
            ARN_EINVAL, "null scale");
  EXPECT_EQ(arn_rmsnorm_fp8(dev8, 64, devf, 9, dev, 64, dev, 1e-6f, 4, 64, ARN_BF16, 0), ARN_EINVAL,
            "fp8 mode");
  EXPECT_EQ(arn_fused_add_rmsnorm_fp8(dev8, 64, devf, ARN_FP8_DYNAMIC, dev, 64, dev, 64, dev, 1e-6f,
                                      0, 64, ARN_BF16, 0), ARN_OK, "fp8 no rows");

  /* descriptor forms */
  arn_norm_args na;
  memset(&na, 0, sizeof(na));
  na.struct_size = sizeof(na);
  na.dtype = ARN_BF16;
  na.out_format = ARN_OUT_16BIT;
  na.out = dev;
  na.out_stride = 64;
  na.x = dev;
  na.x_stride = 64;
  na.eps = 1e-6f;
  na.rows = 0;
  na.hidden = 64;
  EXPECT_EQ(arn_norm(&na), ARN_OK, "arn_norm no rows");
  EXPECT_EQ(arn_norm(NULL), ARN_EINVAL, "arn_norm null");
  na.variance_size = 65;
  na.rows = 2;
  EXPECT_EQ(arn_norm(&na), ARN_EINVAL, "variance size > hidden");
  na.variance_size = 0;
  na.struct_size = 8;
  EXPECT_EQ(arn_norm(&na), ARN_EINVAL, "struct size");

  const void *parts[9] = {dev, dev, dev, dev, dev, dev, dev, dev, dev};
  arn_sum_norm_args sa;
  memset(&sa, 0, sizeof(sa));
  sa.struct_size = sizeof(sa);
  sa.dtype = ARN_BF16;
  sa.out_format = ARN_OUT_16BIT;
  sa.out = dev;
  sa.out_stride = 64;
  sa.parts = parts;
  sa.nparts = 9;
  sa.parts_stride = 64;
  sa.residual = dev;
  sa.residual_stride = 64;
  sa.eps = 1e-6f;
  sa.rows = 2;
  sa.hidden = 64;
  EXPECT_EQ(arn_sum_add_rmsnorm(&sa), ARN_EINVAL, "nine parts");
  sa.nparts = 0;
  EXPECT_EQ(arn_sum_add_rmsnorm(&sa), ARN_EINVAL, "no parts");
  sa.nparts = 8;
  sa.rows = 0;
  EXPECT_EQ(arn_sum_add_rmsnorm(&sa), ARN_OK, "sum no rows");
  EXPECT_EQ(arn_sum_add_rmsnorm(NULL), ARN_EINVAL, "sum null");

  /* SwiGLU */
  EXPECT_EQ(arn_silu_and_mul(dev, 32, NULL, 64, dev, 64, 4, 32, ARN_BF16, 0), ARN_EINVAL, "null gate");
  EXPECT_EQ(arn_silu_and_mul(dev, 32, dev, 16, dev, 64, 4, 32, ARN_BF16, 0), ARN_EINVAL, "gate stride");
  EXPECT_EQ(arn_silu_and_mul(dev, 32, dev, 64, dev, 64, 0, 32, ARN_BF16, 0), ARN_OK, "glu no rows");
  EXPECT_EQ(arn_silu_and_mul_fp8(dev8, 32, NULL, ARN_FP8_DYNAMIC, dev, 64, dev, 64, 4, 32, ARN_BF16,
                                 0), ARN_EINVAL, "glu null scale");

  /* GEMM: size queries, refusals, empty calls */
  EXPECT_EQ(arn_fp8_weight_preshuffled_bytes(33, 200), 3 * 2 * 2048, "shuffled bytes");
  EXPECT_EQ(arn_fp8_weight_preshuffled_bytes(-1, 200), -1, "shuffled bytes n < 0");
  EXPECT_EQ(arn_fp8_weight_preshuffled_bytes(8, 0), -1, "shuffled bytes k 0");
  EXPECT_EQ(arn_fp8_gemm_workspace_bytes(-1, 8, 8) , -1, "workspace m < 0");
  EXPECT_EQ(arn_fp8_gemm_workspace_bytes(64, 4096, 4096) > 0, 1, "workspace bytes");
  EXPECT_EQ(arn_fp8_gemm(dev, 64, ARN_BF16, dev8, 128, devf, 1, dev8, 128, devf, 1, 0, 64, 128, 0),
            ARN_OK, "gemm m 0");
  EXPECT_EQ(arn_fp8_gemm(dev, 64, ARN_BF16, dev8, 128, devf, 1, dev8, 128, devf, 1, 4, 0, 128, 0),
            ARN_OK, "gemm n 0");
  EXPECT_EQ(arn_fp8_gemm(dev, 64, 5, dev8, 128, devf, 1, dev8, 128, devf, 1, 4, 64, 128, 0),
            ARN_EINVAL, "gemm dtype");
  EXPECT_EQ(arn_fp8_gemm(dev, 64, ARN_BF16, dev8, 64, devf, 1, dev8, 128, devf, 1, 4, 64, 128, 0),
            ARN_EINVAL, "gemm lda < k");
  EXPECT_EQ(arn_fp8_gemm(dev, 32, ARN_BF16, dev8, 128, devf, 1, dev8, 128, devf, 1, 4, 64, 128, 0),
            ARN_EINVAL, "gemm ldc < n");
  EXPECT_EQ(arn_fp8_gemm(NULL, 64, ARN_BF16, dev8, 128, devf, 1, dev8, 128, devf, 1, 4, 64, 128, 0),
            ARN_EINVAL, "gemm null c");
  EXPECT_EQ(arn_fp8_gemm_ws(dev, 64, ARN_BF16, dev8, 128, devf, 1, dev8, 128, devf, 1, 4, 64, 128,
                            dev, 16, 0), ARN_EINVAL, "workspace too small");
  EXPECT_EQ(arn_fp8_weight_preshuffle(dev8, NULL, 128, 64, 128, 0), ARN_EINVAL, "shuffle null src");
  EXPECT_EQ(arn_fp8_weight_preshuffle(dev8, dev8, 64, 64, 128, 0), ARN_EINVAL, "shuffle ldb < k");

  /* the no-allocation GEMM: argument and size refusals before any HIP call */
  EXPECT_EQ(arn_fp8_gemm_preshuffled_noalloc(dev, 64, 7, dev8, 128, devf, 1, dev8, devf, 1, 4, 64,
                                             128, 0), ARN_EINVAL, "noalloc bad dtype");
  EXPECT_EQ(arn_fp8_gemm_preshuffled_noalloc(NULL, 64, ARN_BF16, dev8, 128, devf, 1, dev8, devf, 1,
                                             4, 64, 128, 0), ARN_EINVAL, "noalloc null c");
  EXPECT_EQ(arn_fp8_gemm_preshuffled_noalloc(dev, 4033, ARN_BF16, dev8, 128, devf, 1, dev8, devf,
                                             1, 64, 4033, 128, 0), ARN_EUNSUPPORTED,
            "noalloc past its array");
  EXPECT_EQ(arn_fp8_gemm_preshuffled_noalloc(dev, 64, ARN_BF16, dev8, 128, devf, 1, dev8, devf, 1,
                                             0, 64, 128, 0), ARN_OK, "noalloc m = 0");

  /* tuning knobs and the plan buffer */
  EXPECT_EQ(arn_set_tile(3, 3), ARN_EINVAL, "tile not compiled");
  EXPECT_EQ(arn_set_tile(0, 0), ARN_OK, "tile reset");
  EXPECT_EQ(arn_set_gemm_config(3, 4), ARN_EINVAL, "gemm shape not compiled");
  EXPECT_EQ(arn_set_gemm_config(0, 0), ARN_OK, "gemm shape reset");
  EXPECT_EQ(arn_set_gemm_splits(9), ARN_EINVAL, "splits > 8");
  EXPECT_EQ(arn_set_gemm_splits(0), ARN_OK, "splits reset");
  char buf[4];
  const int len = arn_last_plan(buf, sizeof(buf));
  EXPECT_EQ(len >= 0, 1, "plan length");
  EXPECT_EQ(strlen(buf) < sizeof(buf), 1, "plan NUL-terminated");
  EXPECT_EQ(arn_last_plan(buf, 1), len, "plan into one byte");
  EXPECT_EQ(buf[0], 0, "one-byte plan is empty");
  EXPECT_EQ(arn_last_plan(NULL, 0), len, "plan length only");

  /* the plan query: a decode batch of fused rows, its buffer at every
     length, and its refusals (distinct stand-ins, so no aliasing refusal) */
  arn_norm_args q;
  memset(&q, 0, sizeof(q));
  q.struct_size = sizeof(q);
  q.dtype = ARN_BF16;
  q.out_format = ARN_OUT_16BIT;
  q.out = (void *)(uintptr_t)0x1000000;
  q.x = (const void *)(uintptr_t)0x2000000;
  q.residual = (void *)(uintptr_t)0x3000000;
  q.weight = (const void *)(uintptr_t)0x4000000;
  q.out_stride = q.x_stride = q.residual_stride = 8192;
  q.eps = 1e-6f;
  q.rows = 256;
  q.hidden = 8192;
  char pbuf[160];
  EXPECT_EQ(arn_norm_plan(&q, 256, pbuf, sizeof(pbuf)), ARN_OK, "plan query");
  EXPECT_EQ(strcmp(pbuf, "fused_add/bf16/vec8/wpr4/nv4/rpb1/grid256"), 0, "plan of 256 rows");
  char small[4];
  EXPECT_EQ(arn_norm_plan(&q, 256, small, sizeof(small)), ARN_OK, "plan query, short buffer");
  EXPECT_EQ(strlen(small), 3, "short plan truncated and NUL-terminated");
  EXPECT_EQ(arn_norm_plan(&q, 256, NULL, 0), ARN_OK, "plan query, no buffer");
  EXPECT_EQ(arn_norm_plan(&q, 0, pbuf, sizeof(pbuf)), ARN_EINVAL, "no compute units");
  EXPECT_EQ(pbuf[0], 0, "refused plan leaves the buffer empty");
  q.rows = 0;
  EXPECT_EQ(arn_norm_plan(&q, 256, pbuf, sizeof(pbuf)), ARN_OK, "plan of no rows");
  EXPECT_EQ(pbuf[0], 0, "no rows, no plan");
  q.rows = 4;
  q.hidden = 65537;
  q.out_stride = q.x_stride = q.residual_stride = 65537;
  EXPECT_EQ(arn_norm_plan(&q, 256, pbuf, sizeof(pbuf)), ARN_EUNSUPPORTED, "row too long");
  q.residual = (void *)q.x;
  EXPECT_EQ(arn_norm_plan(&q, 256, pbuf, sizeof(pbuf)), ARN_EINVAL, "residual aliases x");
  q.struct_size = 8;
  EXPECT_EQ(arn_norm_plan(&q, 256, pbuf, sizeof(pbuf)), ARN_EINVAL, "descriptor too small");
  EXPECT_EQ(arn_norm_plan(NULL, 256, pbuf, sizeof(pbuf)), ARN_EINVAL, "no descriptor");

  if (failures) {
    fprintf(stderr, "%d check(s) failed\n", failures);
    return 1;
  }
  puts("abi driver: all calls clean");
  return 0;
}
