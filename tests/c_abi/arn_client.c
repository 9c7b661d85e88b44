/*
 * arn_client.c -- a plain C program that drives libarn.so through
 * include/arn.h alone (hipMalloc'd buffers, a HIP stream, no Python, no
 * torch), so the GPU tests can check that the C boundary works by itself.
 *
 *   arn_client norm <plain|fused> <none|static|dynamic> <bf16|fp16> rows hidden stride eps
 *              static_scale variance_size in.bin out.bin
 *       in.bin : x (rows*stride u16), residual (rows*stride u16, fused only),
 *                weight (hidden u16)
 *       out.bin: residual after the call (fused only), out (rows*stride u16,
 *                or rows*stride e4m3 bytes), scales (rows f32, dynamic only)
 *       variance_size 0 calls the named entry point; > 0 goes through arn_norm.
 *   arn_client gemm <rowmajor|preshuffled|preshuffled_ws|preshuffled_noalloc> m n k in.bin
 *              out.bin
 *       in.bin : a (m*k bytes), b (n*k bytes), scale_a (m f32), scale_b (n f32)
 *       out.bin: c (m*n bf16)
 *   arn_client sum <none|dynamic> <bf16|fp16> nparts rows hidden stride eps in.bin out.bin
 *       in.bin : nparts parts (rows*stride u16 each, each copied to its own
 *                buffer), residual (rows*stride u16), weight (hidden u16)
 *       out.bin: residual after the call, out (rows*stride u16, or
 *                rows*stride e4m3 bytes), scales (rows f32, dynamic only)
 *   arn_client glu <none|dynamic> <bf16|fp16> rows d in.bin out.bin
 *       in.bin : gate_up (rows*2d u16: gate in columns [0, d), up in [d, 2d))
 *       out.bin: out (rows*d u16, or rows*d e4m3 bytes), scales (rows f32,
 *                dynamic only)
 *
 * Exit status 0 on success; on any failure a message on stderr and 1.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "arn.h"

#define HIP_OK(call)                                                            \
  do {                                                                          \
    hipError_t e_ = (call);                                                     \
    if (e_ != hipSuccess) {                                                     \
      fprintf(stderr, "%s failed: %s\n", #call, hipGetErrorString(e_));       \
      exit(1);                                                                  \
    }                                                                           \
  } while (0)

#define ARN_OK_(call)                                                           \
  do {                                                                          \
    int s_ = (call);                                                            \
    if (s_ != ARN_OK) {                                                         \
      fprintf(stderr, "%s failed: %s\n", #call, arn_status_str(s_));          \
      exit(1);                                                                  \
    }                                                                           \
  } while (0)

static void *read_file(const char *path, size_t want) {
  FILE *f = fopen(path, "rb");
  if (!f) {
    fprintf(stderr, "cannot open %s\n", path);
    exit(1);
  }
  void *buf = malloc(want ? want : 1);
  if (fread(buf, 1, want, f) != want) {
    fprintf(stderr, "%s: expected %zu bytes\n", path, want);
    exit(1);
  }
  fclose(f);
  return buf;
}

/* Copies size bytes from host memory into a new device buffer. */
static void *to_device(const void *host, size_t size) {
  void *d = NULL;
  HIP_OK(hipMalloc(&d, size ? size : 1));
  if (size) HIP_OK(hipMemcpy(d, host, size, hipMemcpyHostToDevice));
  return d;
}

static void append(FILE *f, const void *dev, size_t size) {
  void *h = malloc(size ? size : 1);
  if (size) HIP_OK(hipMemcpy(h, dev, size, hipMemcpyDeviceToHost));
  if (fwrite(h, 1, size, f) != size) {
    fprintf(stderr, "short write\n");
    exit(1);
  }
  free(h);
}

static int run_norm(char **argv) {
  const int fused = strcmp(argv[0], "fused") == 0;
  const char *fp8 = argv[1];
  const int dtype = strcmp(argv[2], "fp16") == 0 ? ARN_FP16 : ARN_BF16;
  const int64_t rows = atoll(argv[3]), hidden = atoll(argv[4]), stride = atoll(argv[5]);
  const float eps = (float)atof(argv[6]);
  const float static_scale = (float)atof(argv[7]);
  const int64_t variance_size = atoll(argv[8]);
  const int is_fp8 = strcmp(fp8, "none") != 0;
  const int dynamic = strcmp(fp8, "dynamic") == 0;

  const size_t mat16 = (size_t)(rows * stride * 2);
  const size_t in_size = mat16 * (fused ? 2 : 1) + (size_t)hidden * 2;
  uint8_t *in = read_file(argv[9], in_size);
  void *x = to_device(in, mat16);
  void *res = fused ? to_device(in + mat16, mat16) : NULL;
  void *w = to_device(in + mat16 * (fused ? 2 : 1), (size_t)hidden * 2);
  const size_t out_size = is_fp8 ? (size_t)(rows * stride) : mat16;
  void *out = NULL;
  HIP_OK(hipMalloc(&out, out_size ? out_size : 1));
  HIP_OK(hipMemset(out, 0, out_size ? out_size : 1));
  /* static: one dequant scale read; dynamic: `rows` scales written */
  const size_t scale_count = dynamic ? (size_t)rows : 1;
  float *scale = NULL;
  if (dynamic) {
    HIP_OK(hipMalloc((void **)&scale, scale_count * sizeof(float) + 4));
  } else {
    scale = to_device(&static_scale, sizeof(float));
  }
  hipStream_t stream;
  HIP_OK(hipStreamCreate(&stream));

  if (variance_size > 0) {
    arn_norm_args a;
    memset(&a, 0, sizeof(a));
    a.struct_size = sizeof(a);
    a.dtype = dtype;
    a.out_format = !is_fp8 ? ARN_OUT_16BIT : (dynamic ? ARN_OUT_FP8_DYNAMIC : ARN_OUT_FP8_STATIC);
    a.out = out;
    a.out_stride = stride;
    a.scale = scale;
    a.x = x;
    a.x_stride = stride;
    a.residual = res;
    a.residual_stride = stride;
    a.weight = w;
    a.eps = eps;
    a.rows = rows;
    a.hidden = hidden;
    a.variance_size = variance_size;
    a.stream = stream;
    ARN_OK_(arn_norm(&a));
  } else if (!is_fp8 && fused) {
    ARN_OK_(arn_fused_add_rmsnorm(out, stride, x, stride, res, stride, w, eps, rows, hidden,
                                  dtype, stream));
  } else if (!is_fp8) {
    ARN_OK_(arn_rmsnorm(out, stride, x, stride, w, eps, rows, hidden, dtype, stream));
  } else if (fused) {
    ARN_OK_(arn_fused_add_rmsnorm_fp8((uint8_t *)out, stride, scale,
                                      dynamic ? ARN_FP8_DYNAMIC : ARN_FP8_STATIC, x, stride, res,
                                      stride, w, eps, rows, hidden, dtype, stream));
  } else {
    ARN_OK_(arn_rmsnorm_fp8((uint8_t *)out, stride, scale,
                            dynamic ? ARN_FP8_DYNAMIC : ARN_FP8_STATIC, x, stride, w, eps, rows,
                            hidden, dtype, stream));
  }
  HIP_OK(hipStreamSynchronize(stream));
  HIP_OK(hipGetLastError());

  FILE *f = fopen(argv[10], "wb");
  if (!f) {
    fprintf(stderr, "cannot open %s\n", argv[10]);
    return 1;
  }
  if (fused) append(f, res, mat16);
  append(f, out, out_size);
  if (dynamic) append(f, scale, scale_count * sizeof(float));
  fclose(f);
  HIP_OK(hipStreamDestroy(stream));
  return 0;
}

static int run_gemm(char **argv) {
  const int with_ws = strcmp(argv[0], "preshuffled_ws") == 0;
  const int noalloc = strcmp(argv[0], "preshuffled_noalloc") == 0;
  const int pre = with_ws || noalloc || strcmp(argv[0], "preshuffled") == 0;
  const int64_t m = atoll(argv[1]), n = atoll(argv[2]), k = atoll(argv[3]);
  const size_t sa_bytes = (size_t)m * 4, sb_bytes = (size_t)n * 4;
  const size_t in_size = (size_t)(m * k + n * k) + sa_bytes + sb_bytes;
  uint8_t *in = read_file(argv[4], in_size);
  void *a = to_device(in, (size_t)(m * k));
  void *b = to_device(in + m * k, (size_t)(n * k));
  float *sa = to_device(in + m * k + n * k, sa_bytes);
  float *sb = to_device(in + m * k + n * k + sa_bytes, sb_bytes);
  void *c = NULL;
  HIP_OK(hipMalloc(&c, (size_t)(m * n * 2)));
  hipStream_t stream;
  HIP_OK(hipStreamCreate(&stream));
  if (pre) {
    const int64_t bytes = arn_fp8_weight_preshuffled_bytes(n, k);
    if (bytes < 0) {
      fprintf(stderr, "arn_fp8_weight_preshuffled_bytes: invalid shape\n");
      return 1;
    }
    void *bs = NULL;
    HIP_OK(hipMalloc(&bs, (size_t)bytes));
    ARN_OK_(arn_fp8_weight_preshuffle((uint8_t *)bs, (const uint8_t *)b, k, n, k, stream));
    if (with_ws) {
      /* split-K workspace: zero-filled once, reusable afterwards */
      const int64_t ws_bytes = arn_fp8_gemm_workspace_bytes(m, n, k);
      void *ws = NULL;
      HIP_OK(hipMalloc(&ws, (size_t)ws_bytes));
      HIP_OK(hipMemset(ws, 0, (size_t)ws_bytes));
      for (int rep = 0; rep < 2; ++rep) {
        ARN_OK_(arn_fp8_gemm_preshuffled_ws(c, n, ARN_BF16, (const uint8_t *)a, k, sa, 1,
                                            (const uint8_t *)bs, sb, 1, m, n, k, ws,
                                            (size_t)ws_bytes, stream));
      }
      HIP_OK(hipStreamSynchronize(stream));
      HIP_OK(hipFree(ws));
    } else if (noalloc) {
      /* the library's own split-K array: no workspace; twice, as above */
      for (int rep = 0; rep < 2; ++rep) {
        ARN_OK_(arn_fp8_gemm_preshuffled_noalloc(c, n, ARN_BF16, (const uint8_t *)a, k, sa, 1,
                                                 (const uint8_t *)bs, sb, 1, m, n, k, stream));
      }
    } else {
      ARN_OK_(arn_fp8_gemm_preshuffled(c, n, ARN_BF16, (const uint8_t *)a, k, sa, 1,
                                       (const uint8_t *)bs, sb, 1, m, n, k, stream));
    }
    HIP_OK(hipStreamSynchronize(stream));
    HIP_OK(hipFree(bs));
  } else {
    ARN_OK_(arn_fp8_gemm(c, n, ARN_BF16, (const uint8_t *)a, k, sa, 1, (const uint8_t *)b, k, sb,
                         1, m, n, k, stream));
  }
  HIP_OK(hipStreamSynchronize(stream));
  HIP_OK(hipGetLastError());
  FILE *f = fopen(argv[5], "wb");
  if (!f) {
    fprintf(stderr, "cannot open %s\n", argv[5]);
    return 1;
  }
  append(f, c, (size_t)(m * n * 2));
  fclose(f);
  HIP_OK(hipStreamDestroy(stream));
  return 0;
}

static int run_sum(char **argv) {
  const int dynamic = strcmp(argv[0], "dynamic") == 0;
  const int dtype = strcmp(argv[1], "fp16") == 0 ? ARN_FP16 : ARN_BF16;
  const int nparts = atoi(argv[2]);
  const int64_t rows = atoll(argv[3]), hidden = atoll(argv[4]), stride = atoll(argv[5]);
  const float eps = (float)atof(argv[6]);
  if (nparts < 1 || nparts > 8) {
    fprintf(stderr, "nparts must be 1..8\n");
    return 1;
  }
  const size_t mat16 = (size_t)(rows * stride * 2);
  const size_t in_size = mat16 * (size_t)(nparts + 1) + (size_t)hidden * 2;
  uint8_t *in = read_file(argv[7], in_size);
  const void *parts[8];
  for (int p = 0; p < nparts; ++p) parts[p] = to_device(in + mat16 * p, mat16);
  void *res = to_device(in + mat16 * nparts, mat16);
  void *w = to_device(in + mat16 * (nparts + 1), (size_t)hidden * 2);
  const size_t out_size = dynamic ? (size_t)(rows * stride) : mat16;
  void *out = NULL;
  HIP_OK(hipMalloc(&out, out_size ? out_size : 1));
  HIP_OK(hipMemset(out, 0, out_size ? out_size : 1));
  float *scale = NULL;
  if (dynamic) HIP_OK(hipMalloc((void **)&scale, (size_t)rows * sizeof(float) + 4));
  hipStream_t stream;
  HIP_OK(hipStreamCreate(&stream));

  arn_sum_norm_args a;
  memset(&a, 0, sizeof(a));
  a.struct_size = sizeof(a);
  a.dtype = dtype;
  a.out_format = dynamic ? ARN_OUT_FP8_DYNAMIC : ARN_OUT_16BIT;
  a.out = out;
  a.out_stride = stride;
  a.scale = scale;
  a.parts = parts;
  a.nparts = nparts;
  a.parts_stride = stride;
  a.residual = res;
  a.residual_stride = stride;
  a.weight = w;
  a.eps = eps;
  a.rows = rows;
  a.hidden = hidden;
  a.stream = stream;
  ARN_OK_(arn_sum_add_rmsnorm(&a));
  HIP_OK(hipStreamSynchronize(stream));
  HIP_OK(hipGetLastError());

  FILE *f = fopen(argv[8], "wb");
  if (!f) {
    fprintf(stderr, "cannot open %s\n", argv[8]);
    return 1;
  }
  append(f, res, mat16);
  append(f, out, out_size);
  if (dynamic) append(f, scale, (size_t)rows * sizeof(float));
  fclose(f);
  HIP_OK(hipStreamDestroy(stream));
  return 0;
}

static int run_glu(char **argv) {
  const int dynamic = strcmp(argv[0], "dynamic") == 0;
  const int dtype = strcmp(argv[1], "fp16") == 0 ? ARN_FP16 : ARN_BF16;
  const int64_t rows = atoll(argv[2]), d = atoll(argv[3]);
  const size_t in_size = (size_t)(rows * 2 * d * 2);
  uint8_t *in = read_file(argv[4], in_size);
  uint8_t *gu = to_device(in, in_size);
  const size_t out_size = (size_t)(rows * d) * (dynamic ? 1 : 2);
  void *out = NULL;
  HIP_OK(hipMalloc(&out, out_size ? out_size : 1));
  float *scale = NULL;
  if (dynamic) HIP_OK(hipMalloc((void **)&scale, (size_t)rows * sizeof(float) + 4));
  hipStream_t stream;
  HIP_OK(hipStreamCreate(&stream));
  /* gate = the first d columns of each row, up = the next d */
  if (dynamic) {
    ARN_OK_(arn_silu_and_mul_fp8((uint8_t *)out, d, scale, ARN_FP8_DYNAMIC, gu, 2 * d,
                                 gu + d * 2, 2 * d, rows, d, dtype, stream));
  } else {
    ARN_OK_(arn_silu_and_mul(out, d, gu, 2 * d, gu + d * 2, 2 * d, rows, d, dtype, stream));
  }
  HIP_OK(hipStreamSynchronize(stream));
  HIP_OK(hipGetLastError());
  FILE *f = fopen(argv[5], "wb");
  if (!f) {
    fprintf(stderr, "cannot open %s\n", argv[5]);
    return 1;
  }
  append(f, out, out_size);
  if (dynamic) append(f, scale, (size_t)rows * sizeof(float));
  fclose(f);
  HIP_OK(hipStreamDestroy(stream));
  return 0;
}

int main(int argc, char **argv) {
  if (arn_abi_version() != ARN_ABI_VERSION) {
    fprintf(stderr, "libarn ABI %d, header %d\n", arn_abi_version(), ARN_ABI_VERSION);
    return 1;
  }
  if (argc == 13 && strcmp(argv[1], "norm") == 0) return run_norm(argv + 2);
  if (argc == 8 && strcmp(argv[1], "gemm") == 0) return run_gemm(argv + 2);
  if (argc == 11 && strcmp(argv[1], "sum") == 0) return run_sum(argv + 2);
  if (argc == 8 && strcmp(argv[1], "glu") == 0) return run_glu(argv + 2);
  fprintf(stderr, "usage: see the comment at the top of arn_client.c\n");
  return 1;
}
