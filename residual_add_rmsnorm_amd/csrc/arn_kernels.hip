// arn_kernels.hip -- gfx950 (CDNA4) kernels for residual-add + RMSNorm
// (+ OCP e4m3 output).  Compiled once per operator kind and dtype
// (-DARN_KIND=0..5 -DARN_DT=0|1); each unit exports one table of tiles.
//
// The method: per row, r = x + residual (stored back, rounded to 16 bits),
// y = r / sqrt(mean(r^2) + eps) * w (Zhang & Sennrich 2019, eq. 4), then
// optionally an e4m3 cast -- the three steps the first kernel of "Custom
// CUDA kernels juice Llama 3.1 405B on AMD MI300X" (paragraph 2) fuses into
// one pass.  That kernel targeted MI300X; this one is laid out for gfx950:
//
//  * The op moves 7-8 bytes per element and does a handful of VALU ops per
//    element, so HBM bandwidth bounds it; there is no contraction and no
//    MFMA.  Each row is read once and written once.
//  * Lane l of the T = 64*WPR threads that share a row owns the VEC-element
//    vectors l, l+T, l+2T, ... (VEC = 8 x 16-bit = 128-bit loads, so one
//    wave instruction moves 1 KiB of contiguous row).  The whole row stays
//    in VGPRs between the sum-of-squares pass and the output pass.
//  * WPR = 1 (row per wave) reduces with DPP row ops + 4 readlanes and no
//    LDS or barrier; WPR > 1 (row per workgroup) adds one LDS exchange of
//    per-wave partials behind one barrier.  Sum and, for dynamic FP8, the
//    max |r*w| travel together, so dynamic FP8 costs no extra barrier:
//    max |y| = max |r*w| * inv because inv > 0.
//  * Reductions use a fixed order, so results are bitwise reproducible.
//  * e4m3 codes come from the packed gfx950 v_cvt_pk_fp8_f32 (OCP format
//    on this target) after an explicit fmed3 clamp to +-448.
//  * x and out may alias: every element is loaded before the reduction and
//    stored after it by the same lane, so nothing is marked __restrict__.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "arn_device.h"
#include "arn_internal.h"

#if !defined(ARN_KIND) || !defined(ARN_DT)
#error "compile with -DARN_KIND=<0..5> -DARN_DT=<0|1> [-DARN_SUM=1]"
#endif
#if !defined(ARN_SUM)
#define ARN_SUM 0
#endif

namespace arn {
namespace {

using namespace dev;

// ---------------------------------------------------------------------------
// The kernel.
// ---------------------------------------------------------------------------
template <int DT, int KIND, int VEC, int NV, int WPR, int RPB, bool SUM>
__global__ __launch_bounds__(64 * WPR * RPB) void row_kernel(const Args a) {
  constexpr bool kRes = (KIND & 1) != 0;
  constexpr bool kStatic = (KIND & 2) != 0;
  constexpr bool kDynamic = (KIND & 4) != 0;
  constexpr bool kFp8 = kStatic || kDynamic;
  constexpr int kTPR = 64 * WPR;                     // threads per row
  constexpr uint32_t kStep16 = kTPR * VEC * 2;       // bytes between a lane's vectors
  constexpr uint32_t kStep8 = kTPR * VEC;            // same, e4m3 output

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  // kTPR is a multiple of 64, so every lane of a wave has the same row;
  // readfirstlane lets the compiler keep row addresses in SGPRs.
  const int rib = __builtin_amdgcn_readfirstlane(tid / kTPR);  // row within the block
  const int t = tid - rib * kTPR;                              // thread within the row
  const uint32_t off16 = (uint32_t)t * (VEC * 2);
  const uint32_t off8 = (uint32_t)t * VEC;
  const uint32_t row_bytes16 = (uint32_t)a.hidden * 2u;
  const uint32_t row_bytes8 = (uint32_t)a.hidden;

  // One block handles RPB consecutive rows (the host splits launches whose
  // row count exceeds the grid limit).  A row past the end gets
  // num_records = 0, so its lanes still take part in the reduction but
  // read zeros and write nothing.
  const int64_t row = (int64_t)blockIdx.x * RPB + rib;
  const bool active = row < a.rows;
  const int64_t arow = active ? row : 0;
  const uint32_t n16 = active ? row_bytes16 : 0u;

  const __amdgpu_buffer_rsrc_t xrs =
      row_rsrc(static_cast<const uint16_t*>(a.x) + arow * a.x_stride, n16);
  __amdgpu_buffer_rsrc_t rrs = xrs;
  if constexpr (kRes) rrs = row_rsrc(static_cast<const uint16_t*>(a.res) + arow * a.res_stride, n16);

  __shared__ float red_sum[WPR * RPB];  // one slot per wave
  __shared__ float red_max[WPR * RPB];

  {
    // 1. Load the row: x (and residual) into registers.  Vectors past the
    //    row end read as zero.
    Raw<VEC> xr[NV];
    Raw<VEC> rr[NV];
    if constexpr (SUM) {
      // All-reduce form: every part's vectors are loaded, then x is the
      // fp32 sum in rank order (part 0 first), rounded once to 16 bits --
      // the value an all-reduce would hand to the unfused norm.
      Raw<VEC> pr[kMaxParts][NV];
#pragma unroll
      for (int g = 0; g < kMaxParts; ++g) {
        if (g < a.nparts) {
          const __amdgpu_buffer_rsrc_t prs =
              row_rsrc(static_cast<const uint16_t*>(a.parts[g]) + arow * a.x_stride, n16);
#pragma unroll
          for (int k = 0; k < NV; ++k) pr[g][k] = load16<VEC, kCacheStream>(prs, off16 + k * kStep16);
        }
      }
#pragma unroll
      for (int k = 0; k < NV; ++k) {
        if constexpr (kRes) rr[k] = load16<VEC, kCacheStream>(rrs, off16 + k * kStep16);
      }
#pragma unroll
      for (int k = 0; k < NV; ++k) {
        float acc[VEC];
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc[e] = elem<DT, VEC>(pr[0][k], e);
#pragma unroll
        for (int g = 1; g < kMaxParts; ++g) {
          if (g < a.nparts) {
#pragma unroll
            for (int e = 0; e < VEC; ++e) acc[e] = acc[e] + elem<DT, VEC>(pr[g][k], e);
          }
        }
        xr[k] = pack<DT, VEC>(acc);
      }
    } else {
#pragma unroll
      for (int k = 0; k < NV; ++k) {
        xr[k] = load16<VEC, kCacheStream>(xrs, off16 + k * kStep16);
        if constexpr (kRes) rr[k] = load16<VEC, kCacheStream>(rrs, off16 + k * kStep16);
      }
    }
    // The weight (shared by all rows; an L2 hit after the first blocks).
    Raw<VEC> wr[NV];
    if (a.w != nullptr) {
      const __amdgpu_buffer_rsrc_t wrs = row_rsrc(a.w, row_bytes16);
#pragma unroll
      for (int k = 0; k < NV; ++k) wr[k] = load16<VEC, kCacheDefault>(wrs, off16 + k * kStep16);
    } else {
#pragma unroll
      for (int k = 0; k < NV; ++k) wr[k] = ones<DT, VEC>();
    }
    float qmul = 0.0f;
    if constexpr (kStatic) qmul = 1.0f / *a.scale;

    // 2. r = x + residual in fp32, rounded to 16 bits and stored back;
    //    sum of squares of the rounded r over the first var_cols channels
    //    (all of them unless the variance size is overridden), and max |r*w|
    //    for dynamic FP8.  Zero-filled vectors add nothing and their stores
    //    are dropped.
    if constexpr (kRes) {
#pragma unroll
      for (int k = 0; k < NV; ++k) {
        float f[VEC];
#pragma unroll
        for (int e = 0; e < VEC; ++e) f[e] = elem<DT, VEC>(xr[k], e) + elem<DT, VEC>(rr[k], e);
        xr[k] = pack<DT, VEC>(f);
        store16<VEC>(xr[k], rrs, off16 + k * kStep16);
      }
    }
    float ss = 0.0f;
    float mx = 0.0f;
    if (a.var_cols == a.hidden) {
#pragma unroll
      for (int k = 0; k < NV; ++k) {
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          const float rf = elem<DT, VEC>(xr[k], e);
          ss = __builtin_fmaf(rf, rf, ss);
        }
      }
    } else {
#pragma unroll
      for (int k = 0; k < NV; ++k) {
        const int col0 = (t + k * kTPR) * VEC;
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          const float rf = elem<DT, VEC>(xr[k], e);
          ss = __builtin_fmaf(rf, col0 + e < a.var_cols ? rf : 0.0f, ss);
        }
      }
    }
    if constexpr (kDynamic) {
#pragma unroll
      for (int k = 0; k < NV; ++k) {
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          mx = fmaxf(mx, fabsf(elem<DT, VEC>(xr[k], e) * elem<DT, VEC>(wr[k], e)));
        }
      }
    }

    // 3. Row reduction: wave, then (row per workgroup) across waves via LDS.
    ss = wave_sum(ss);
    if constexpr (kDynamic) mx = wave_max(mx);
    if constexpr (WPR > 1) {
      if (lane == 0) {
        red_sum[wave] = ss;
        if constexpr (kDynamic) red_max[wave] = mx;
      }
      __syncthreads();
      ss = 0.0f;
      mx = 0.0f;
#pragma unroll
      for (int i = 0; i < WPR; ++i) {
        ss += red_sum[rib * WPR + i];
        if constexpr (kDynamic) mx = fmaxf(mx, red_max[rib * WPR + i]);
      }
    }
    const float inv = rsqrtf(__builtin_fmaf(ss, a.inv_var, a.eps));

    if constexpr (kDynamic) {
      const float amax = mx * inv;
      qmul = amax > 0.0f ? 448.0f / amax : 0.0f;
      if (active && t == 0) a.scale[row] = amax / 448.0f;
    }

    // 4. y = r * inv * w, stored as 16 bits or as e4m3 codes.
    if constexpr (kFp8) {
      const __amdgpu_buffer_rsrc_t ors = row_rsrc(
          static_cast<uint8_t*>(a.out) + arow * a.out_stride, active ? row_bytes8 : 0u);
#pragma unroll
      for (int k = 0; k < NV; ++k) {
        float y[VEC];
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          y[e] = elem<DT, VEC>(xr[k], e) * inv * elem<DT, VEC>(wr[k], e) * qmul;
        }
        store8<VEC>(pack_fp8<VEC>(y), ors, off8 + k * kStep8);
      }
    } else {
      const __amdgpu_buffer_rsrc_t ors =
          row_rsrc(static_cast<uint16_t*>(a.out) + arow * a.out_stride, n16);
#pragma unroll
      for (int k = 0; k < NV; ++k) {
        float y[VEC];
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          y[e] = elem<DT, VEC>(xr[k], e) * inv * elem<DT, VEC>(wr[k], e);
        }
        store16<VEC>(pack<DT, VEC>(y), ors, off16 + k * kStep16);
      }
    }
  }
}

constexpr int rows_per_block(int wpr) { return wpr >= 4 ? 1 : 4 / wpr; }

}  // namespace
}  // namespace arn

#define ARN_TILE(VEC, WPR, NV)                                                              \
  {VEC, WPR, NV, arn::rows_per_block(WPR),                                                 \
   (const void*)&arn::row_kernel<ARN_DT, ARN_KIND, VEC, NV, WPR, arn::rows_per_block(WPR), \
                                 ARN_SUM != 0>}

#if ARN_SUM
// All-reduce form: up to kMaxParts inputs held per vector, so at most four
// vectors per lane.
static const arn::Tile kTiles[] = {
    ARN_TILE(8, 4, 1), ARN_TILE(8, 4, 2), ARN_TILE(8, 8, 1), ARN_TILE(8, 8, 2),
    ARN_TILE(8, 16, 1), ARN_TILE(8, 16, 2), ARN_TILE(8, 16, 4),
    ARN_TILE(4, 16, 2), ARN_TILE(4, 16, 4), ARN_TILE(2, 16, 4), ARN_TILE(1, 16, 4),
};

extern const arn::TileTable ARN_SUM_TABLE_NAME(ARN_KIND, ARN_DT) = {
    kTiles, (int)(sizeof(kTiles) / sizeof(kTiles[0]))};
#else
static const arn::Tile kTiles[] = {
    // 128-bit accesses (hidden % 8 == 0, 16-byte aligned rows)
    ARN_TILE(8, 1, 2), ARN_TILE(8, 1, 4), ARN_TILE(8, 1, 8), ARN_TILE(8, 1, 16),
    ARN_TILE(8, 2, 2), ARN_TILE(8, 2, 4), ARN_TILE(8, 2, 8),
    ARN_TILE(8, 4, 1), ARN_TILE(8, 4, 2), ARN_TILE(8, 4, 3), ARN_TILE(8, 4, 4), ARN_TILE(8, 4, 8),
    ARN_TILE(8, 8, 1), ARN_TILE(8, 8, 2), ARN_TILE(8, 8, 4), ARN_TILE(8, 8, 8),
    ARN_TILE(8, 16, 1), ARN_TILE(8, 16, 2), ARN_TILE(8, 16, 4), ARN_TILE(8, 16, 8),
    // narrower accesses for rows that are not 16-byte aligned
    ARN_TILE(4, 1, 4), ARN_TILE(4, 4, 4), ARN_TILE(4, 16, 4), ARN_TILE(4, 16, 16),
    ARN_TILE(2, 1, 4), ARN_TILE(2, 4, 4), ARN_TILE(2, 16, 4), ARN_TILE(2, 16, 16),
    ARN_TILE(1, 1, 4), ARN_TILE(1, 4, 4), ARN_TILE(1, 16, 4), ARN_TILE(1, 16, 16),
};

extern const arn::TileTable ARN_TABLE_NAME(ARN_KIND, ARN_DT) = {
    kTiles, (int)(sizeof(kTiles) / sizeof(kTiles[0]))};
#endif
