// arn_probe.hip -- plain streaming kernels that measure the HBM bandwidth a
// given mix of read and write streams reaches on this GPU, as the practical
// ceiling for a bandwidth-bound operator moving the same byte mix.  No
// arithmetic beyond what keeps the loads live; the same access style as the
// operator kernels (128-bit buffer loads and stores bounded by the stream
// length, non-temporal cache policy), grid-stride loop.
//
// A mix is R read streams of 16 bytes per element, W16 write streams of 16
// bytes and W8 write streams of 8 bytes per element:
//   fused add + RMSNorm, 16-bit out:   R 2, W16 2   (reads 4H, writes 4H bytes per row)
//   fused add + RMSNorm + e4m3:        R 2, W16 1, W8 1   (4H : 3H)
//   SwiGLU + e4m3:                     R 2, W8 1   (4d : d)
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "arn_probe.h"

namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

constexpr int kNt = 2;  // non-temporal

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes,
                                           0x00020000);
}

template <int B, int R, int W16, int W8>
__global__ __launch_bounds__(B) void stream_kernel(const void* a, const void* b, void* c, void* d,
                                                   int64_t n) {
  const auto ra = rsrc(a, (uint32_t)(n * 16));
  const auto rb = rsrc(b, (uint32_t)(n * 16));
  const auto rc = rsrc(c, (uint32_t)(n * 16));
  const auto rd = rsrc(d, (uint32_t)(n * (W16 == 2 ? 16 : 8)));
  const int64_t stride = (int64_t)gridDim.x * B;
  u32x4 keep = {0u, 0u, 0u, 0u};
  for (int64_t i = (int64_t)blockIdx.x * B + threadIdx.x; i < n; i += stride) {
    const uint32_t off = (uint32_t)i * 16u;
    u32x4 va = {(uint32_t)i, 1u, 2u, 3u};
    u32x4 vb = va;
    if constexpr (R >= 1) va = __builtin_amdgcn_raw_buffer_load_b128(ra, (int)off, 0, kNt);
    if constexpr (R >= 2) vb = __builtin_amdgcn_raw_buffer_load_b128(rb, (int)off, 0, kNt);
    const u32x4 s = va + vb;
    // 16-byte streams go to c, then d; an 8-byte stream goes to d.
    if constexpr (W16 >= 1) __builtin_amdgcn_raw_buffer_store_b128(s, rc, (int)off, 0, kNt);
    if constexpr (W16 >= 2) __builtin_amdgcn_raw_buffer_store_b128(va ^ vb, rd, (int)off, 0, kNt);
    if constexpr (W8 >= 1) {
      const u32x2 h = {s.x ^ s.z, s.y ^ s.w};
      __builtin_amdgcn_raw_buffer_store_b64(h, rd, (int)(off / 2u), 0, kNt);
    }
    if constexpr (W16 == 0 && W8 == 0) keep ^= s;
  }
  // Read-only mix: keep the loads live with a store no real input triggers.
  if constexpr (W16 == 0 && W8 == 0) {
    if (keep.x == 0x9e3779b9u && keep.y == 0x7f4a7c15u && keep.z == 0xf39cc060u) {
      __builtin_amdgcn_raw_buffer_store_b128(keep, rc, 0, 0, 0);
    }
  }
}

// Many read streams (the all-reduce form reads every rank's part and the
// residual): R streams of 16 bytes per element summed, written to c (16
// bytes) and d (16 or 8 bytes per element).
struct ManyArgs {
  const void* src[16];
  void* c;
  void* d;
  int64_t n;
};

template <int B, int R, int W16, int W8>
__global__ __launch_bounds__(B) void many_kernel(const ManyArgs p) {
  __amdgpu_buffer_rsrc_t rs[R];
#pragma unroll
  for (int r = 0; r < R; ++r) rs[r] = rsrc(p.src[r], (uint32_t)(p.n * 16));
  const auto rc = rsrc(p.c, (uint32_t)(p.n * 16));
  const auto rd = rsrc(p.d, (uint32_t)(p.n * (W16 == 2 ? 16 : 8)));
  const int64_t stride = (int64_t)gridDim.x * B;
  for (int64_t i = (int64_t)blockIdx.x * B + threadIdx.x; i < p.n; i += stride) {
    const uint32_t off = (uint32_t)i * 16u;
    u32x4 v[R];
#pragma unroll
    for (int r = 0; r < R; ++r) v[r] = __builtin_amdgcn_raw_buffer_load_b128(rs[r], (int)off, 0, kNt);
    u32x4 s = v[0];
#pragma unroll
    for (int r = 1; r < R; ++r) s += v[r];
    if constexpr (W16 >= 1) __builtin_amdgcn_raw_buffer_store_b128(s, rc, (int)off, 0, kNt);
    if constexpr (W16 >= 2) __builtin_amdgcn_raw_buffer_store_b128(s ^ v[0], rd, (int)off, 0, kNt);
    if constexpr (W8 >= 1) {
      const u32x2 h = {s.x ^ s.z, s.y ^ s.w};
      __builtin_amdgcn_raw_buffer_store_b64(h, rd, (int)(off / 2u), 0, kNt);
    }
  }
}

template <int R, int W16, int W8>
hipError_t launch_many(int block, const ManyArgs& a, int grid, hipStream_t stream) {
  void* params[] = {const_cast<ManyArgs*>(&a)};
  const void* fn = nullptr;
  if (block == 256) fn = (const void*)&many_kernel<256, R, W16, W8>;
  if (block == 512) fn = (const void*)&many_kernel<512, R, W16, W8>;
  if (block == 1024) fn = (const void*)&many_kernel<1024, R, W16, W8>;
  return hipLaunchKernel(fn, dim3((unsigned)grid), dim3((unsigned)block), params, 0, stream);
}

// The fused norm's traffic with the row structure kept: each block owns G
// consecutive rows (row pitch `stride` bytes, `len` bytes used, len <= 16
// KiB), and for every row reads x and the residual and writes the residual
// back in place and the output.  512 threads, two 16-byte vectors per
// thread per row and stream; buffer records end at `len`, so a shorter row
// drops the excess loads and stores.  The order of a block's accesses is
// the variable:
//   MODE 0  row by row: load x_g, r_g, store r_g, o_g (the operator's order)
//   MODE 1  all loads of the G rows, then each row's two stores
//   MODE 2  all loads, then every residual store, then every output store
//   MODE 3  one row ahead: load row g+1 before storing row g
struct RowsArgs {
  const char* x;
  char* res;
  char* out;
  int64_t rows;
  int64_t stride;
  uint32_t len;
};

template <int G, int MODE>
__global__ __launch_bounds__(512) void rows_kernel(const RowsArgs p) {
  constexpr int kNv = 2;
  const uint32_t off = threadIdx.x * 16u;
  auto rs = [&](const char* base, int64_t row) {
    return rsrc(base + row * p.stride, row < p.rows ? p.len : 0u);
  };
  const int64_t row0 = (int64_t)blockIdx.x * G;
  u32x4 xv[G][kNv], rv[G][kNv];
  auto load_row = [&](int g) {
#pragma unroll
    for (int k = 0; k < kNv; ++k) {
      xv[g][k] = __builtin_amdgcn_raw_buffer_load_b128(rs(p.x, row0 + g), (int)(off + k * 8192u), 0, kNt);
      rv[g][k] = __builtin_amdgcn_raw_buffer_load_b128(rs(p.res, row0 + g), (int)(off + k * 8192u), 0, kNt);
    }
  };
  auto store_res = [&](int g) {
#pragma unroll
    for (int k = 0; k < kNv; ++k) {
      __builtin_amdgcn_raw_buffer_store_b128(xv[g][k] + rv[g][k], rs(p.res, row0 + g),
                                             (int)(off + k * 8192u), 0, kNt);
    }
  };
  auto store_out = [&](int g) {
#pragma unroll
    for (int k = 0; k < kNv; ++k) {
      __builtin_amdgcn_raw_buffer_store_b128(xv[g][k] ^ rv[g][k], rs(p.out, row0 + g),
                                             (int)(off + k * 8192u), 0, kNt);
    }
  };
  if constexpr (MODE == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      load_row(g);
      store_res(g);
      store_out(g);
    }
  } else if constexpr (MODE == 1) {
#pragma unroll
    for (int g = 0; g < G; ++g) load_row(g);
#pragma unroll
    for (int g = 0; g < G; ++g) {
      store_res(g);
      store_out(g);
    }
  } else if constexpr (MODE == 2) {
#pragma unroll
    for (int g = 0; g < G; ++g) load_row(g);
#pragma unroll
    for (int g = 0; g < G; ++g) store_res(g);
#pragma unroll
    for (int g = 0; g < G; ++g) store_out(g);
  } else {
    load_row(0);
#pragma unroll
    for (int g = 0; g < G; ++g) {
      if (g + 1 < G) load_row(g + 1);
      store_res(g);
      store_out(g);
    }
  }
}

template <int G>
const void* rows_fn(int mode) {
  switch (mode) {
    case 0: return (const void*)&rows_kernel<G, 0>;
    case 1: return (const void*)&rows_kernel<G, 1>;
    case 2: return (const void*)&rows_kernel<G, 2>;
    case 3: return (const void*)&rows_kernel<G, 3>;
    default: return nullptr;
  }
}

// Does nothing: the cost of a launch itself, the floor under any small
// kernel's time per call.
__global__ __launch_bounds__(1024) void empty_kernel() {}

template <int R, int W16, int W8>
hipError_t launch(int block, const void* a, const void* b, void* c, void* d, int64_t n,
                  int grid, hipStream_t stream) {
  void* params[] = {&a, &b, &c, &d, &n};
  const void* fn = nullptr;
  if (block == 256) fn = (const void*)&stream_kernel<256, R, W16, W8>;
  if (block == 512) fn = (const void*)&stream_kernel<512, R, W16, W8>;
  if (block == 1024) fn = (const void*)&stream_kernel<1024, R, W16, W8>;
  return hipLaunchKernel(fn, dim3((unsigned)grid), dim3((unsigned)block), params, 0, stream);
}

}  // namespace

extern "C" int arn_probe_stream(int reads, int writes16, int writes8, const void* a,
                                const void* b, void* c, void* d, int64_t n, int grid, int block,
                                hipStream_t stream) {
  if (n <= 0 || n > (int64_t(1) << 27) || grid <= 0 || grid > (1 << 24)) return 1;
  if (block != 256 && block != 512 && block != 1024) return 1;
  if ((reads >= 1 && !a) || (reads >= 2 && !b) || !c) return 1;
  if ((writes16 >= 2 || writes8 >= 1) && !d) return 1;
  hipError_t e;
  if (reads == 1 && writes16 == 0 && writes8 == 0) {
    e = launch<1, 0, 0>(block, a, b, c, d, n, grid, stream);
  } else if (reads == 0 && writes16 == 1 && writes8 == 0) {
    e = launch<0, 1, 0>(block, a, b, c, d, n, grid, stream);
  } else if (reads == 1 && writes16 == 1 && writes8 == 0) {
    e = launch<1, 1, 0>(block, a, b, c, d, n, grid, stream);
  } else if (reads == 2 && writes16 == 2 && writes8 == 0) {
    e = launch<2, 2, 0>(block, a, b, c, d, n, grid, stream);
  } else if (reads == 2 && writes16 == 1 && writes8 == 1) {
    e = launch<2, 1, 1>(block, a, b, c, d, n, grid, stream);
  } else if (reads == 2 && writes16 == 0 && writes8 == 1) {
    e = launch<2, 0, 1>(block, a, b, c, d, n, grid, stream);
  } else {
    return 2;
  }
  return e == hipSuccess ? 0 : 3;
}

extern "C" int arn_probe_empty(int grid, int block, hipStream_t stream) {
  if (grid <= 0 || grid > (1 << 24) || block <= 0 || block > 1024) return 1;
  return hipLaunchKernel((const void*)&empty_kernel, dim3((unsigned)grid), dim3((unsigned)block),
                         nullptr, 0, stream) == hipSuccess
             ? 0
             : 3;
}

extern "C" int arn_probe_stream_many(int reads, int writes16, int writes8,
                                     const void* const* srcs, void* c, void* d, int64_t n,
                                     int grid, int block, hipStream_t stream) {
  if (n <= 0 || n > (int64_t(1) << 27) || grid <= 0 || grid > (1 << 24)) return 1;
  if (block != 256 && block != 512 && block != 1024) return 1;
  if (!srcs || !c || !d || reads < 1 || reads > 16) return 1;
  ManyArgs a;
  for (int r = 0; r < 16; ++r) a.src[r] = r < reads ? srcs[r] : nullptr;
  for (int r = 0; r < reads; ++r) {
    if (!a.src[r]) return 1;
  }
  a.c = c;
  a.d = d;
  a.n = n;
  hipError_t e;
  if (reads == 9 && writes16 == 2 && writes8 == 0) {
    e = launch_many<9, 2, 0>(block, a, grid, stream);
  } else if (reads == 9 && writes16 == 1 && writes8 == 1) {
    e = launch_many<9, 1, 1>(block, a, grid, stream);
  } else {
    return 2;
  }
  return e == hipSuccess ? 0 : 3;
}

extern "C" int arn_probe_rows(int mode, int rows_per_block, const void* x, void* res, void* out,
                              int64_t rows, int64_t row_bytes, int64_t stride_bytes,
                              hipStream_t stream) {
  if (!x || !res || !out || rows <= 0 || row_bytes <= 0 || row_bytes > 16384 ||
      row_bytes % 16 != 0 || stride_bytes < row_bytes || mode < 0 || mode > 3) {
    return 1;
  }
  const void* fn = nullptr;
  if (rows_per_block == 1) fn = rows_fn<1>(mode);
  if (rows_per_block == 2) fn = rows_fn<2>(mode);
  if (rows_per_block == 4) fn = rows_fn<4>(mode);
  if (!fn) return 2;
  const int64_t grid = (rows + rows_per_block - 1) / rows_per_block;
  if (grid > (int64_t(1) << 24) || (rows - 1) * stride_bytes + row_bytes > (int64_t(1) << 40)) {
    return 1;
  }
  RowsArgs a;
  a.x = static_cast<const char*>(x);
  a.res = static_cast<char*>(res);
  a.out = static_cast<char*>(out);
  a.rows = rows;
  a.stride = stride_bytes;
  a.len = (uint32_t)row_bytes;
  void* params[] = {&a};
  return hipLaunchKernel(fn, dim3((unsigned)grid), dim3(512u), params, 0, stream) == hipSuccess
             ? 0
             : 3;
}
