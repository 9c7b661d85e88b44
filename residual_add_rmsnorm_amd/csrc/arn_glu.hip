// arn_glu.hip -- gfx950 kernels for the SwiGLU activation fused with its
// output cast: out = silu(gate) * up, as 16 bits or as OCP e4m3 codes with a
// static per-tensor or dynamic per-row scale.  Compiled once per output mode
// and dtype (-DARN_GLU_MODE=0..2 -DARN_DT=0|1).
//
// The second kernel of "Custom CUDA kernels juice Llama 3.1 405B on AMD
// MI300X" (paragraph 2) merges SwiGLU with the FP8 cast; SwiGLU is
// Swish_1(xW) * (xV) (Shazeer, "GLU Variants Improve Transformer", 2020),
// with the two projections arriving as the gate and up halves.  Like the
// norm kernels this moves a few bytes per element and does a few dozen VALU
// ops per element, so it streams at HBM speed:
//  * rows of WPR waves, VEC-element 128-bit buffer accesses bounded by the
//    row length (ragged ends need no branches);
//  * sigmoid in the form that cannot overflow: e = exp(-|g|),
//    sigmoid(g) = 1/(1+e) for g >= 0 and e/(1+e) below, so silu stays
//    accurate for large negative g;
//  * dynamic e4m3 keeps the row's y in VGPRs while max |y| is reduced (DPP
//    across the wave, LDS across waves), then scales and converts.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "arn_device.h"
#include "arn_internal.h"

#if !defined(ARN_GLU_MODE) || !defined(ARN_DT)
#error "compile with -DARN_GLU_MODE=<0..2> -DARN_DT=<0|1>"
#endif

namespace arn {
namespace {

using namespace dev;

// silu(g) = g * sigmoid(g) with sigmoid(g) = 1/(1+e) for g >= 0 and e/(1+e)
// below, e = exp(-|g|) <= 1, so nothing overflows.  e is computed as
// 2^(64 - |g| log2(e)) * 2^-64 with the hardware exp2 (v_exp_f32) and the
// reciprocal with v_rcp_f32 (both about 1 ulp): the exp2 result stays a
// normal number until |g| > 190, and the exact power-of-two rescale lets
// large negative gates keep their tiny silu values, including fp32
// subnormal ones.  Shifting the argument by 64 costs about 2^-18 relative
// in e, far below the 16-bit output's rounding.  About ten VALU ops per
// element, which keeps the kernel memory-bound.
__device__ __forceinline__ float silu(float g) {
  const float e =
      __builtin_amdgcn_exp2f(__builtin_fmaf(-fabsf(g), 1.44269504088896341f, 64.0f)) * 0x1p-64f;
  const float r = __builtin_amdgcn_rcpf(1.0f + e);
  return g * (g >= 0.0f ? r : e * r);
}

template <int DT, int MODE, int VEC, int NV, int WPR, int RPB>
__global__ __launch_bounds__(64 * WPR * RPB) void glu_kernel(const GluArgs a) {
  constexpr bool kStatic = MODE == kGluStatic;
  constexpr bool kDynamic = MODE == kGluDynamic;
  constexpr bool kFp8 = kStatic || kDynamic;
  constexpr int kTPR = 64 * WPR;
  constexpr uint32_t kStep16 = kTPR * VEC * 2;
  constexpr uint32_t kStep8 = kTPR * VEC;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int rib = __builtin_amdgcn_readfirstlane(tid / kTPR);
  const int t = tid - rib * kTPR;
  const uint32_t off16 = (uint32_t)t * (VEC * 2);
  const uint32_t off8 = (uint32_t)t * VEC;
  const uint32_t row_bytes16 = (uint32_t)a.d * 2u;

  const int64_t row = (int64_t)blockIdx.x * RPB + rib;
  const bool active = row < a.rows;
  const int64_t arow = active ? row : 0;
  const uint32_t n16 = active ? row_bytes16 : 0u;
  const __amdgpu_buffer_rsrc_t grs =
      row_rsrc(static_cast<const uint16_t*>(a.gate) + arow * a.gate_stride, n16);
  const __amdgpu_buffer_rsrc_t urs =
      row_rsrc(static_cast<const uint16_t*>(a.up) + arow * a.up_stride, n16);

  Raw<VEC> gr[NV], ur[NV];
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    gr[k] = load16<VEC, kCacheStream>(grs, off16 + k * kStep16);
    ur[k] = load16<VEC, kCacheStream>(urs, off16 + k * kStep16);
  }

  float y[NV][VEC];
  float mx = 0.0f;
#pragma unroll
  for (int k = 0; k < NV; ++k) {
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      y[k][e] = silu(elem<DT, VEC>(gr[k], e)) * elem<DT, VEC>(ur[k], e);
      if constexpr (kDynamic) mx = fmaxf(mx, fabsf(y[k][e]));
    }
  }

  float qmul = 1.0f;
  if constexpr (kStatic) qmul = 1.0f / *a.scale;
  if constexpr (kDynamic) {
    __shared__ float red_max[WPR * RPB];
    mx = wave_max(mx);
    if constexpr (WPR > 1) {
      if (lane == 0) red_max[wave] = mx;
      __syncthreads();
      mx = 0.0f;
#pragma unroll
      for (int i = 0; i < WPR; ++i) mx = fmaxf(mx, red_max[rib * WPR + i]);
    }
    qmul = mx > 0.0f ? 448.0f / mx : 0.0f;
    if (active && t == 0) a.scale[row] = mx / 448.0f;
  }

  if constexpr (kFp8) {
    const __amdgpu_buffer_rsrc_t ors = row_rsrc(
        static_cast<uint8_t*>(a.out) + arow * a.out_stride, active ? (uint32_t)a.d : 0u);
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      float v[VEC];
#pragma unroll
      for (int e = 0; e < VEC; ++e) v[e] = y[k][e] * qmul;
      store8<VEC>(pack_fp8<VEC>(v), ors, off8 + k * kStep8);
    }
  } else {
    const __amdgpu_buffer_rsrc_t ors =
        row_rsrc(static_cast<uint16_t*>(a.out) + arow * a.out_stride, n16);
#pragma unroll
    for (int k = 0; k < NV; ++k) store16<VEC>(pack<DT, VEC>(y[k]), ors, off16 + k * kStep16);
  }
}

constexpr int rows_per_block(int wpr) { return wpr >= 4 ? 1 : 4 / wpr; }

}  // namespace
}  // namespace arn

#define ARN_GTILE(VEC, WPR, NV)                                                          \
  {VEC, WPR, NV, arn::rows_per_block(WPR),                                               \
   (const void*)&arn::glu_kernel<ARN_DT, ARN_GLU_MODE, VEC, NV, WPR, arn::rows_per_block(WPR)>}

static const arn::Tile kGluTiles[] = {
    ARN_GTILE(8, 1, 2), ARN_GTILE(8, 1, 4), ARN_GTILE(8, 2, 2), ARN_GTILE(8, 2, 4),
    ARN_GTILE(8, 4, 1), ARN_GTILE(8, 4, 2), ARN_GTILE(8, 4, 4),
    ARN_GTILE(8, 8, 1), ARN_GTILE(8, 8, 2), ARN_GTILE(8, 8, 4),
    ARN_GTILE(8, 16, 1), ARN_GTILE(8, 16, 2), ARN_GTILE(8, 16, 4), ARN_GTILE(8, 16, 8),
    ARN_GTILE(4, 1, 4), ARN_GTILE(4, 4, 4), ARN_GTILE(4, 16, 4), ARN_GTILE(4, 16, 16),
    ARN_GTILE(2, 1, 4), ARN_GTILE(2, 4, 4), ARN_GTILE(2, 16, 4), ARN_GTILE(2, 16, 16),
    ARN_GTILE(1, 1, 4), ARN_GTILE(1, 4, 4), ARN_GTILE(1, 16, 4), ARN_GTILE(1, 16, 16),
};

extern const arn::TileTable ARN_GLU_TABLE_NAME(ARN_GLU_MODE, ARN_DT) = {
    kGluTiles, (int)(sizeof(kGluTiles) / sizeof(kGluTiles[0]))};
