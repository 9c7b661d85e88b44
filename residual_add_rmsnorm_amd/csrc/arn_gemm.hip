// arn_gemm.hip -- gfx950 "skinny" GEMM on OCP e4m3 codes:
//     C[m][n] = sa(m) * sb(n) * sum_k A[m][k] * B[n][k]
// with A the e4m3 activations (M x K, per-row or per-tensor dequant scale,
// e.g. the codes and scales the fused norm / SwiGLU kernels write) and B an
// e4m3 weight stored out-feature major (N x K, per-row or per-tensor
// scale).  The third kernel of "Custom CUDA kernels juice Llama 3.1 405B on
// AMD MI300X" (paragraph 2) is a GEMM tuned for the small-batch shapes of
// decoding; this is that contraction built for gfx950.  Compiled once per
// output dtype (-DARN_DT=0|1).
//
// Decode GEMMs stream the weight: with M <= 64 rows of activations the
// bytes of B dominate and the kernel is HBM-bound, so the layout serves the
// weight stream:
//  * v_mfma_f32_16x16x128_f8f6f4 (e4m3 x e4m3 -> fp32): each lane brings 32
//    bytes of one row of A and of B for a 128-wide k step.  Row-major
//    operands are loaded as whole 128-byte rows and put into operand order
//    through LDS (see aoff below); the pre-shuffled weight arrives in
//    operand order.  The k order inside an MFMA is the same for both
//    operands, and a dot product does not depend on it.
//  * a block owns a (16 MT) x (16 NT) output tile and splits K over WAVES
//    waves in interleaved 128-wide steps (the block reads each weight row
//    front to back); A tiles are reused across the NT weight tiles of a
//    step.  Partial tiles are summed through LDS in a fixed order, so the
//    result is deterministic; the dequant scales are applied at the store.
//  * operands are read with bounded buffer loads: rows past M or N read as
//    zero, and a k step past K is given an out-of-range offset.
//  * weights may come pre-shuffled into MFMA tile order (every load then
//    reads 1 KiB contiguous), and K may be split across blocks through a
//    caller workspace when N alone gives too few blocks for the CUs.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "arn_device.h"
#include "arn_gemm.h"

#if !defined(ARN_DT)
#error "compile with -DARN_DT=<0|1>"
#endif

namespace arn {
namespace {

using namespace dev;

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Byte offset past any slice a launch addresses (the host keeps slices
// under 2 GiB): a 16-byte load there reads zeros.
constexpr uint32_t kOutOfRange = 0xFFFFFF00u;

// Cache policy sc1: a load coherent across the XCDs (agent scope), the
// policy a relaxed agent-scope atomic load compiles to.
constexpr int kCacheDeviceScope = 16;

// A lane's 32 bytes of one 128-byte k step come from two 16-byte pieces:
// bytes [16 q, 16 q + 16) and [64 + 16 q, 64 + 16 q + 16) for lane group q.
// Each load instruction then reads 64 contiguous bytes of every row it
// touches.  The MFMA pairs A and B bytes by their position in the lane, and
// both operands use this same map, so the dot product is unchanged.  Each
// piece gets its own offset, out of range when it lies past K.
template <int CP>
__device__ __forceinline__ i32x8 load32(__amdgpu_buffer_rsrc_t r, uint32_t lo, uint32_t hi) {
  const u32x4 a = __builtin_amdgcn_raw_buffer_load_b128(r, (int)lo, 0, CP);
  const u32x4 b = __builtin_amdgcn_raw_buffer_load_b128(r, (int)hi, 0, CP);
  i32x8 v;
  v[0] = (int)a.x;
  v[1] = (int)a.y;
  v[2] = (int)a.z;
  v[3] = (int)a.w;
  v[4] = (int)b.x;
  v[5] = (int)b.y;
  v[6] = (int)b.z;
  v[7] = (int)b.w;
  return v;
}

template <int DT, int MT, int NT, int WAVES, bool PRE>
__global__ __launch_bounds__(64 * WAVES) __attribute__((amdgpu_waves_per_eu(1, 4)))
void gemm_fp8_kernel(const GemmArgs g) {
  constexpr int kTile = MT * NT * 256;  // outputs per block

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r16 = lane & 15;  // operand row within a 16-row tile
  const int kq = lane >> 4;   // 32-byte quarter of a 128-wide k step

  const int64_t n0 = (int64_t)blockIdx.x * 16 * NT;
  const int64_t n_here = (g.n - n0) < 16 * NT ? (g.n - n0) : 16 * NT;
  const int nsteps = (int)((g.k + 127) / 128);
  // This block's k steps: all of them, or one split's share.
  const int s_begin = (int)blockIdx.y * g.steps_per_split;
  const int s_end = min(nsteps, s_begin + g.steps_per_split);
  const __amdgpu_buffer_rsrc_t ars = row_rsrc(g.a, (uint32_t)(g.m * g.lda));
  // Row-major weight: this block's rows.  Pre-shuffled weight: the launch's
  // panel, k-step major -- step s of column tile T at (s * ntiles + T) * 2 KiB,
  // so the blocks of a launch, moving through K at about the same pace,
  // read one compact region of the weight at a time rather than one
  // stream each.
  const int64_t ntiles = (g.n + 15) / 16;
  const uint32_t step_bytes = (uint32_t)(ntiles * 2048);
  const __amdgpu_buffer_rsrc_t brs =
      PRE ? row_rsrc(g.b, (uint32_t)(ntiles * nsteps * 2048))
          : row_rsrc(static_cast<const uint8_t*>(g.b) + n0 * g.ldb, (uint32_t)(n_here * g.ldb));

  // Row-major operands.  The MFMA layout puts one operand row in every 16th
  // lane, so a load that fills operand registers directly touches 16 rows
  // (16 cache lines, half of each) per instruction, where a load of the
  // pre-shuffled weight touches 8 whole lines.  So every row-major tile --
  // A always, the weight unless pre-shuffled -- is loaded as whole 128-byte
  // rows (lane l: row l / 8, bytes 16 (l % 8); two loads per 16-row tile)
  // and put into operand order through the wave's own LDS slice (rows
  // padded to 144 bytes, so that the operand reads -- 16 rows at one column
  // -- fall in distinct banks).
  constexpr int kRowP = 144;
  constexpr int kStage = 16 * kRowP;  // LDS bytes per wave: one tile at a time
  uint32_t aoff[MT], boff[NT];
  bool b_in[NT];  // pre-shuffled: the column tile exists (the last group may be ragged)
#pragma unroll
  for (int i = 0; i < MT; ++i) {
    aoff[i] = (uint32_t)((i * 16 + (lane >> 3)) * g.lda) + 16u * (lane & 7);
  }
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    b_in[t] = !PRE || n0 / 16 + t < ntiles;
    boff[t] = PRE ? (uint32_t)((n0 / 16 + t) * 2048) + 16u * lane
                  : (uint32_t)((t * 16 + (lane >> 3)) * g.ldb) + 16u * (lane & 7);
  }

  f32x4 acc[MT][NT];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[i][t] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};

  // K steps of 128 are dealt to the waves round-robin.  Two register sets
  // ping-pong: the loads of a wave's next step are in flight while the MFMAs
  // of its current step run, and no register copy forces an early wait.  A
  // step outside this block's range reads zeros through out-of-range
  // offsets (no memory traffic), so the loop always runs whole pairs.
  auto load_step = [&](int s, i32x8 (&bq)[NT], i32x8 (&aq)[MT]) {
    const uint32_t kb = (uint32_t)s * 128u;
    const bool in_s = s < s_end;
    // Whole rows: rows 0-7 of each tile in [0..3], rows 8-15 in [4..7]
    // (permute reorders them); K % 16 == 0, so each 16-byte piece is wholly
    // inside or outside K.
    const bool row_in = in_s && kb + 16u * (lane & 7) < (uint32_t)g.k;
#pragma unroll
    for (int i = 0; i < MT; ++i) {
      aq[i] = load32<kCacheDefault>(ars, row_in ? aoff[i] + kb : kOutOfRange,
                                    row_in ? aoff[i] + kb + 8u * (uint32_t)g.lda : kOutOfRange);
    }
    if constexpr (PRE) {
      // Pre-shuffled: a 2 KiB tile per (column tile, k step), read as two
      // 1 KiB contiguous halves; lane l gets bytes [32 q, 32 q + 32) of
      // k step s for row l % 16 (q = l / 16).  K is padded with zero codes
      // to whole steps in the shuffled copy.
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const bool in = in_s && b_in[t];
        const uint32_t o = boff[t] + (uint32_t)s * step_bytes;
        bq[t] = load32<kCacheStream>(brs, in ? o : kOutOfRange, in ? o + 1024u : kOutOfRange);
      }
    } else {
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        bq[t] = load32<kCacheStream>(brs, row_in ? boff[t] + kb : kOutOfRange,
                                     row_in ? boff[t] + kb + 8u * (uint32_t)g.ldb : kOutOfRange);
      }
    }
  };
  // The LDS of the block: the waves' staging slices during the k loop, then
  // the partial tiles of the cross-wave sum.
  constexpr int kLdsBytes =
      WAVES * kStage > WAVES * kTile * 4 ? WAVES * kStage : WAVES * kTile * 4;
  __shared__ __attribute__((aligned(16))) uint8_t lds[kLdsBytes];
  uint8_t* const stage = lds + wave * kStage;
  // One tile into the MFMA operand layout: lane l = r + 16 q gets row r's
  // bytes [32 q, 32 q + 32) of the step (pre-shuffled weight) or [16 q, +16)
  // and [64 + 16 q, +16) (row-major weight), the in-lane k order of the
  // weight operand.  Only this wave touches its slice, and the LDS executes
  // a wave's accesses in order, so the next tile may overwrite the slice
  // right behind the reads, and no barrier is needed.
  auto permute = [&](const i32x8& raw, i32x8& out) {
    const u32x4 lo = {(uint32_t)raw[0], (uint32_t)raw[1], (uint32_t)raw[2], (uint32_t)raw[3]};
    const u32x4 hi = {(uint32_t)raw[4], (uint32_t)raw[5], (uint32_t)raw[6], (uint32_t)raw[7]};
    uint8_t* dst = stage + (lane >> 3) * kRowP + 16 * (lane & 7);
    *reinterpret_cast<u32x4*>(dst) = lo;
    *reinterpret_cast<u32x4*>(dst + 8 * kRowP) = hi;
    const uint8_t* src = stage + r16 * kRowP;
    const u32x4 x0 = *reinterpret_cast<const u32x4*>(src + (PRE ? 32 * kq : 16 * kq));
    const u32x4 x1 = *reinterpret_cast<const u32x4*>(src + (PRE ? 32 * kq + 16 : 64 + 16 * kq));
    out = (i32x8){(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w,
                  (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
  };
  auto mma = [&](const i32x8 (&b_raw)[NT], const i32x8 (&a_raw)[MT]) {
    i32x8 aq[MT], bq[NT];
#pragma unroll
    for (int i = 0; i < MT; ++i) permute(a_raw[i], aq[i]);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      if constexpr (PRE) {
        bq[t] = b_raw[t];
      } else {
        permute(b_raw[t], bq[t]);
      }
    }
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int t = 0; t < NT; ++t)
        acc[i][t] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(aq[i], bq[t], acc[i][t], 0,
                                                                     0, 0, 0, 0, 0);
  };
  // Each thread stores the same tile elements e = threadIdx.x + 64 WAVES i
  // at the end.  Their dequant scales are all requested before any is used,
  // so the block waits for one round trip rather than one per element: with
  // few elements per thread before the k loop (the latency hides behind it),
  // otherwise right after the loop (it overlaps the cross-wave sum), where
  // holding them does not cost loop registers.
  constexpr int kPer = (kTile + 64 * WAVES - 1) / (64 * WAVES);
  constexpr bool kEarlyScales = kPer <= 4;
  float pre_sa[kPer], pre_sb[kPer];
  auto fetch_scales = [&]() {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int e = threadIdx.x + 64 * WAVES * i;
      const int tile = e >> 8;
      const int64_t gm = (int64_t)(tile / NT) * 16 + ((e >> 4) & 15);
      const int64_t gn = n0 + (int64_t)(tile % NT) * 16 + (e & 15);
      // Unconditional loads from clamped (always valid) indices, then a
      // select: no branch, so no wait between the loads.
      const bool out = e < kTile && gm < g.m && gn < g.n;
      const int64_t ia = (g.a_per_row && out) ? gm : 0;
      const int64_t ib = (g.b_per_row && out) ? gn : 0;
      const float sa = g.scale_a[ia];
      const float sb = g.scale_b[ib];
      pre_sa[i] = out ? sa : 0.0f;
      pre_sb[i] = out ? sb : 0.0f;
    }
  };
  if constexpr (kEarlyScales) fetch_scales();

  // The scheduling barriers keep the compiler from sinking each load next
  // to its use (which would serialise load and MFMA again).
  i32x8 b0[NT], a0[MT], b1[NT], a1[MT];
  load_step(s_begin + wave, b0, a0);
  for (int s = s_begin + wave; s < s_end; s += 2 * WAVES) {
    load_step(s + WAVES, b1, a1);
    __builtin_amdgcn_sched_barrier(0);
    mma(b0, a0);
    __builtin_amdgcn_sched_barrier(0);
    load_step(s + 2 * WAVES, b0, a0);
    __builtin_amdgcn_sched_barrier(0);
    mma(b1, a1);
    __builtin_amdgcn_sched_barrier(0);
  }

  // Sum the WAVES partial tiles.  In a 16x16 MFMA result, lane l holds
  // rows 4*(l/16) .. 4*(l/16)+3 of column l%16.
  if constexpr (!kEarlyScales) fetch_scales();
  __syncthreads();  // every wave is done with its staging slice
  float* const part = reinterpret_cast<float*>(lds);
  __shared__ int last_split;
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        part[wave * kTile + ((i * NT + t) * 16 + 4 * kq + j) * 16 + r16] = acc[i][t][j];
  __syncthreads();

  // Each thread owns the same tile elements e = threadIdx.x + 64 WAVES i in
  // every phase below.
  float sum[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int e = threadIdx.x + 64 * WAVES * i;
    sum[i] = 0.0f;
    if (e < kTile) {
#pragma unroll
      for (int w = 0; w < WAVES; ++w) sum[i] += part[w * kTile + e];
    }
  }

  if (g.splits > 1) {
    // Publish this split's partial tile; the block that completes the
    // tile's count sums all splits in split order (so the result does not
    // depend on which block finishes last).  The blocks of one tile may run
    // on different XCDs, whose L2 caches are not coherent with each other,
    // so the partials move with agent-scope (sc1) stores and loads, which
    // are coherent across XCDs, rather than plain accesses made visible by
    // agent-scope fences (each such fence writes back or invalidates a
    // whole L2, which costs far more than the split saves).  Every thread
    // waits for its stores to complete before the barrier that precedes the
    // count, so a block that sees the count complete reads finished tiles.
    float* tile_part = g.partial + (size_t)blockIdx.x * g.splits * kTile;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int e = threadIdx.x + 64 * WAVES * i;
      if (e < kTile) {
        __hip_atomic_store(tile_part + (size_t)blockIdx.y * kTile + e, sum[i], __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == 0) {
      const int done = __hip_atomic_fetch_add(g.counters + blockIdx.x, 1, __ATOMIC_RELAXED,
                                              __HIP_MEMORY_SCOPE_AGENT);
      last_split = done == g.splits - 1;
    }
    __syncthreads();
    if (!last_split) return;
    // The same agent-scope (sc1) loads as relaxed atomic loads, written as
    // buffer loads so that the kPer loads of a split are all in flight
    // before the first is used; each element still adds the splits in
    // split order.
    const __amdgpu_buffer_rsrc_t prs =
        row_rsrc(tile_part, (uint32_t)(g.splits * kTile * (int)sizeof(float)));
#pragma unroll
    for (int i = 0; i < kPer; ++i) sum[i] = 0.0f;
    for (int sp = 0; sp < g.splits; ++sp) {
      float v[kPer];
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        const int e = threadIdx.x + 64 * WAVES * i;
        const uint32_t off = e < kTile ? (uint32_t)((sp * kTile + e) * 4) : kOutOfRange;
        v[i] = __builtin_bit_cast(
            float, __builtin_amdgcn_raw_buffer_load_b32(prs, (int)off, 0, kCacheDeviceScope));
      }
#pragma unroll
      for (int i = 0; i < kPer; ++i) sum[i] += v[i];
    }
    // Leave the counter at zero for the next call (ordered before the next
    // kernel on the stream by the kernel boundary).
    if (threadIdx.x == 0) {
      __hip_atomic_store(g.counters + blockIdx.x, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }

#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int e = threadIdx.x + 64 * WAVES * i;
    if (e >= kTile) continue;
    const int tile = e >> 8;
    const int row = (e >> 4) & 15;
    const int col = e & 15;
    const int64_t gm = (int64_t)(tile / NT) * 16 + row;
    const int64_t gn = n0 + (int64_t)(tile % NT) * 16 + col;
    if (gm < g.m && gn < g.n) {
      const float sa = pre_sa[i];
      const float sb = pre_sb[i];
      const float v = sum[i] * sa * sb;
      static_cast<uint16_t*>(g.c)[gm * g.ldc + gn] = (uint16_t)(pack2<DT>(v, 0.0f) & 0xFFFFu);
    }
  }
}

// Pre-shuffle: one thread per 16-byte piece of the shuffled weight.  The
// shuffled copy holds ceil(n/16) column tiles x ceil(k/128) k steps of
// 2 KiB, in panels of p.panel_tiles column tiles, k-step major inside a
// panel (arn_internal.h).  In a tile, piece p (16 bytes) holds, for row
// r = p % 16 of the column tile and lane group q = (p % 64) / 16, k bytes
// [32 q + 16 (p / 64), +16) of the step -- so that lane l of a load of
// bytes [16 l, 16 l + 16) and of [1024 + 16 l, +16) receives the 32 bytes
// [32 q, 32 q + 32) of row l % 16 that the MFMA operand layout wants.
// Rows past n and k bytes past k are zero codes.  Any row stride works;
// aligned rows are read 16 bytes at a time.
__global__ __launch_bounds__(256) void preshuffle_kernel(const PreshuffleArgs p) {
  const int64_t piece = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t total = p.ntiles * p.nsteps * 128;
  if (piece >= total) return;
  const int64_t tile = piece / 128;  // position of the 2 KiB tile in the copy
  const int pp = (int)(piece % 128);
  const int64_t panel = tile / (p.panel_tiles * p.nsteps);
  const int64_t first = panel * p.panel_tiles;  // first column tile of the panel
  const int64_t width = p.ntiles - first < p.panel_tiles ? p.ntiles - first : p.panel_tiles;
  const int64_t in_panel = tile - first * p.nsteps;
  const int64_t s = in_panel / width;
  const int64_t nt = first + in_panel % width;
  const int64_t row = nt * 16 + (pp % 16);
  const int64_t k0 = s * 128 + 32 * ((pp % 64) / 16) + 16 * (pp / 64);
  u32x4 v = {0u, 0u, 0u, 0u};
  if (row < p.n) {
    const uint8_t* src = static_cast<const uint8_t*>(p.src) + row * p.ldb;
    if (p.aligned && k0 + 16 <= p.k) {
      v = *reinterpret_cast<const u32x4*>(src + k0);  // b and ldb 16-byte aligned
    } else {
      uint8_t b[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) b[i] = (k0 + i < p.k) ? src[k0 + i] : 0;
      v = __builtin_bit_cast(u32x4, b);
    }
  }
  reinterpret_cast<u32x4*>(p.dst)[piece] = v;
}

}  // namespace
}  // namespace arn

#define ARN_GEMM_CFG(MT, NT, WAVES)                                             \
  {MT, NT, WAVES, (const void*)&arn::gemm_fp8_kernel<ARN_DT, MT, NT, WAVES, false>, \
   (const void*)&arn::gemm_fp8_kernel<ARN_DT, MT, NT, WAVES, true>}

static const arn::GemmCfg kGemmCfgs[] = {
    ARN_GEMM_CFG(1, 4, 4), ARN_GEMM_CFG(1, 4, 8), ARN_GEMM_CFG(1, 4, 16),
    ARN_GEMM_CFG(1, 2, 4), ARN_GEMM_CFG(1, 2, 8), ARN_GEMM_CFG(1, 2, 16),
    ARN_GEMM_CFG(1, 1, 4), ARN_GEMM_CFG(1, 1, 8), ARN_GEMM_CFG(1, 1, 16),
    ARN_GEMM_CFG(2, 4, 4), ARN_GEMM_CFG(2, 4, 8),
    ARN_GEMM_CFG(2, 2, 4), ARN_GEMM_CFG(2, 2, 8), ARN_GEMM_CFG(2, 2, 16),
    ARN_GEMM_CFG(2, 1, 4), ARN_GEMM_CFG(2, 1, 8), ARN_GEMM_CFG(2, 1, 16),
    ARN_GEMM_CFG(4, 4, 4), ARN_GEMM_CFG(4, 4, 8),
    ARN_GEMM_CFG(4, 2, 4), ARN_GEMM_CFG(4, 2, 8),
    ARN_GEMM_CFG(4, 1, 4), ARN_GEMM_CFG(4, 1, 8), ARN_GEMM_CFG(4, 1, 16),
};

extern const arn::GemmTable ARN_GEMM_TABLE_NAME(ARN_DT) = {
    kGemmCfgs, (int)(sizeof(kGemmCfgs) / sizeof(kGemmCfgs[0]))};

#if ARN_DT == 0
extern const void* const arn_preshuffle_fn = (const void*)&arn::preshuffle_kernel;
#endif
