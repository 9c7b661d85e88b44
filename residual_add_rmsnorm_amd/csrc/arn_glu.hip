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
//    sigmoid(g) = 1/(1+e) for g >= 0 and e/(1+e) below; a lane with a gate
//    at or below -80, where e nears fp32's subnormal range, forms its
//    outputs in fp64 instead;
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
// normal number until |g| > 190 and the power-of-two rescale is exact while
// e is a normal fp32 number, |g| < 87.3.  (Below that e is subnormal and
// loses bits; the kernel sends gates at or below -80 to silu_mul_f64.)
// Shifting the argument by 64 costs about 2^-18 relative in e, far below
// the 16-bit output's rounding.  About ten VALU ops per element, which
// keeps the kernel memory-bound.
__device__ __forceinline__ float silu(float g) {
  const float e =
      __builtin_amdgcn_exp2f(__builtin_fmaf(-fabsf(g), 1.44269504088896341f, 64.0f)) * 0x1p-64f;
  const float r = __builtin_amdgcn_rcpf(1.0f + e);
  return g * (g >= 0.0f ? r : e * r);
}

// silu(g) * u in fp64, for rows whose outputs leave fp32's range and for
// lanes holding a gate at or below -80.
// exp(-|g|) = 2^-(n + fr) with n = floor(|g| log2 e) and fr in [0, 1): the
// hardware exp2 of -fr, then an exact fp64 ldexp by -n, so gates far below
// -87 (where silu() underflows in fp32) keep their value down to fp64's
// range.  The product with u is exact up to fp64 rounding.  n - a must
// subtract the rounded a (exact, as both are fp32 values within a factor of
// two of each other or a < 1): contracting |g| log2 e into it as an fma
// would leave the rounding error of a, which for |g| near 2^66 is about
// 2^43, in the exponent.
[[maybe_unused]] __device__ __forceinline__ double silu_mul_f64(float g, float u) {
#pragma clang fp contract(off)
  const float a = fabsf(g) * 1.44269504088896341f;
  const float n = floorf(a);
  const double e = __builtin_ldexp((double)__builtin_amdgcn_exp2f(n - a), -(int)fminf(n, 2000.0f));
  const double r = (double)__builtin_amdgcn_rcpf(1.0f + (float)e);
  return (double)g * (g >= 0.0f ? r : e * r) * (double)u;
}

// Elementwise unsigned max of the 16-bit halves of a running word and of
// every 32-bit word of a raw vector (v_pk_max_u16).
template <int VEC>
__device__ __forceinline__ uint32_t max_u16x2(uint32_t acc, const Raw<VEC>& r) {
  typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));
  auto mx = [](uint32_t a, uint32_t b) {
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(u16x2, a),
                                                                  __builtin_bit_cast(u16x2, b)));
  };
  if constexpr (VEC == 1) {
    return mx(acc, (uint32_t)r);
  } else if constexpr (VEC == 2) {
    return mx(acc, r);
  } else {
#pragma unroll
    for (int i = 0; i < VEC / 2; ++i) acc = mx(acc, r[i]);
    return acc;
  }
}

template <int DT, int MODE, int VEC, int NV, int WPR, int RPB>
__global__ __launch_bounds__(64 * WPR * RPB) void glu_kernel(const GluArgs a) {
  constexpr bool kStatic = MODE == kGluStatic;
  constexpr bool kDynamic = MODE == kGluDynamic;
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

  // A lane holding a gate at or below -80 forms its outputs in fp64
  // instead: there exp(-|g|) nears the bottom of fp32's normal range, and
  // past -87.3 silu() keeps only an fp32 subnormal's few bits, which an up
  // value as small as 2^5 lifts into a bf16 output's range.  The bits of a
  // negative 16-bit float order like its magnitude and lie above every
  // positive one, so one packed unsigned max over the raw gate words finds
  // such a gate (and -inf or a negative NaN, which the fp64 form also
  // gives as the definition does).  The branch is skipped when no lane of
  // the wave needs it, and one element's fp64 temporaries are live at a
  // time (as in the wide path below).
  uint32_t gtop = 0;  // running max of the gate words, taken vector by vector
  auto deep = [&]() __attribute__((always_inline)) {
    const uint32_t m = __builtin_elementwise_max(gtop & 0xFFFFu, gtop >> 16);
    return m >= (DT == kBF16 ? 0xC2A0u : 0xD500u);  // -80 in bf16 / fp16
  };
  // The fp64 outputs of a lane, one vector at a time, from inputs read
  // again (L2 or HBM), so the usual path retires its raw registers.
  auto deep_outputs = [&](auto&& use) __attribute__((always_inline)) {
    float prev = 0.0f;
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      asm volatile("" ::: "memory");
      const Raw<VEC> g2 = load16<VEC, kCacheStream>(grs, off16 + k * kStep16);
      const Raw<VEC> u2 = load16<VEC, kCacheStream>(urs, off16 + k * kStep16);
      float v[VEC];
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        float g = elem<DT, VEC>(g2, e), u = elem<DT, VEC>(u2, e);
        asm volatile("" : "+v"(g), "+v"(u) : "v"(prev));
        v[e] = prev = (float)silu_mul_f64(g, u);
      }
      use(k, v);
    }
  };

  if constexpr (!kDynamic) {
    // 16-bit or static e4m3 outputs: each lane stores its own vectors.
    float y[NV][VEC];
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      gtop = max_u16x2<VEC>(gtop, gr[k]);
#pragma unroll
      for (int e = 0; e < VEC; ++e) y[k][e] = silu(elem<DT, VEC>(gr[k], e)) * elem<DT, VEC>(ur[k], e);
    }
    float qmul = 1.0f;
    if constexpr (kStatic) qmul = 1.0f / *a.scale;
    const __amdgpu_buffer_rsrc_t ors =
        kStatic ? row_rsrc(static_cast<uint8_t*>(a.out) + arow * a.out_stride,
                           active ? (uint32_t)a.d : 0u)
                : row_rsrc(static_cast<uint16_t*>(a.out) + arow * a.out_stride, n16);
    auto emit = [&](int k, float (&v)[VEC]) __attribute__((always_inline)) {
      if constexpr (kStatic) {
#pragma unroll
        for (int e = 0; e < VEC; ++e) v[e] *= qmul;
        store8<VEC>(pack_fp8<VEC>(v), ors, off8 + k * kStep8);
      } else {
        store16<VEC>(pack<DT, VEC>(v), ors, off16 + k * kStep16);
      }
    };
#pragma unroll
    for (int k = 0; k < NV; ++k) emit(k, y[k]);
    // A lane with a deep gate stores its vectors a second time, from the
    // fp64 form; the same lane's later store to an address is the one that
    // stays.  The usual path is left as it would be without the check.
    if (__builtin_expect(deep(), 0)) deep_outputs(emit);
  } else {
    // Dynamic e4m3 keeps the row's outputs while max|y| is reduced.
    float y[NV][VEC];
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      gtop = max_u16x2<VEC>(gtop, gr[k]);
#pragma unroll
      for (int e = 0; e < VEC; ++e) y[k][e] = silu(elem<DT, VEC>(gr[k], e)) * elem<DT, VEC>(ur[k], e);
    }
    if (__builtin_expect(deep(), 0)) {
      deep_outputs([&](int k, float (&v)[VEC]) __attribute__((always_inline)) {
#pragma unroll
        for (int e = 0; e < VEC; ++e) y[k][e] = v[e];
      });
    }
    float mx = 0.0f;
#pragma unroll
    for (int k = 0; k < NV; ++k) {
#pragma unroll
      for (int e = 0; e < VEC; ++e) mx = fmaxf(mx, fabsf(y[k][e]));
    }
    __shared__ float red_max[WPR * RPB];
    mx = wave_max(mx);
    if constexpr (WPR > 1) {
      if (lane == 0) red_max[wave] = mx;
      __syncthreads();
      mx = 0.0f;
#pragma unroll
      for (int i = 0; i < WPR; ++i) mx = fmaxf(mx, red_max[rib * WPR + i]);
    }
    // code = e4m3(y / scale) with scale = max|y| / 448 rounded to fp32.  A
    // row whose max|y| is not in [2^-96, 2^128) ("wide": a product silu(g)
    // * u overflowed, or every output is tiny or zero) forms its outputs
    // again in fp64 from the inputs (read a second time; they are never
    // written), one vector at a time and twice -- once for the max, once
    // for the codes -- so the branch holds few registers.  Its codes divide
    // by the stored scale in fp64 (infinite quotients where the scale
    // rounded to zero, zero where it overflowed, as y / scale gives).  Rows
    // sharing a barrier enter together; for a row that did not need it the
    // fp64 outputs round to the same codes within the one-step rule.
    const bool wide = !(mx >= 0x1p-96f && mx <= 3.4028234e38f);
    bool enter_w = wide;
    if constexpr (WPR > 1 && RPB > 1) {
      enter_w = false;
#pragma unroll
      for (int rr = 0; rr < RPB; ++rr) {
        float m = 0.0f;
#pragma unroll
        for (int i = 0; i < WPR; ++i) m = fmaxf(m, red_max[rr * WPR + i]);
        enter_w = enter_w || !(m >= 0x1p-96f && m <= 3.4028234e38f);
      }
    }
    if (enter_w) {
      __shared__ double red_wide[WPR * RPB];
      double m2 = 0.0;
#pragma unroll
      for (int k = 0; k < NV; ++k) {
        asm volatile("" ::: "memory");  // one vector's reloads at a time
        const Raw<VEC> g2 = load16<VEC, kCacheStream>(grs, off16 + k * kStep16);
        const Raw<VEC> u2 = load16<VEC, kCacheStream>(urs, off16 + k * kStep16);
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          // One element at a time: its inputs wait on the running max, so
          // the fp64 temporaries of several elements are never live together.
          float g = elem<DT, VEC>(g2, e), u = elem<DT, VEC>(u2, e);
          asm volatile("" : "+v"(g), "+v"(u) : "v"(m2));
          m2 = fmax(m2, fabs(silu_mul_f64(g, u)));
        }
      }
      m2 = wave_max_f64(m2);
      if constexpr (WPR > 1) {
        if (lane == 0) red_wide[wave] = m2;
        __syncthreads();
        m2 = 0.0;
#pragma unroll
        for (int i = 0; i < WPR; ++i) m2 = fmax(m2, red_wide[rib * WPR + i]);
      }
      const float s = (float)(m2 * (1.0 / 448.0));
      if (active && t == 0) a.scale[row] = s;
      const double qd = m2 > 0.0 ? 1.0 / (double)s : 0.0;  // an all-zero row: codes 0
      const __amdgpu_buffer_rsrc_t ors = row_rsrc(
          static_cast<uint8_t*>(a.out) + arow * a.out_stride, active ? (uint32_t)a.d : 0u);
#pragma unroll
      for (int k = 0; k < NV; ++k) {
        asm volatile("" ::: "memory");
        const Raw<VEC> g2 = load16<VEC, kCacheStream>(grs, off16 + k * kStep16);
        const Raw<VEC> u2 = load16<VEC, kCacheStream>(urs, off16 + k * kStep16);
        float v[VEC];
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          float g = elem<DT, VEC>(g2, e), u = elem<DT, VEC>(u2, e);
          if (e > 0) asm volatile("" : "+v"(g), "+v"(u) : "v"(v[e - 1]));
          v[e] = (float)(silu_mul_f64(g, u) * qd);
        }
        store8<VEC>(pack_fp8<VEC>(v), ors, off8 + k * kStep8);
      }
      return;
    }
    // Any other row: max|y| in [2^-96, 2^128), so 448 / max|y| and the
    // scale max|y| / 448 are normal fp32 numbers (the reciprocal of mx / 448
    // in [2^-105, 2^120) by the hardware's 1-ulp v_rcp_f32), and an output
    // that lost low bits below 2^-126 is off by less than 2^-54 of the max.
    const float qmul = __builtin_amdgcn_rcpf(mx * (1.0f / 448.0f));
    if (active && t == 0) a.scale[row] = mx * (1.0f / 448.0f);
    const __amdgpu_buffer_rsrc_t ors = row_rsrc(
        static_cast<uint8_t*>(a.out) + arow * a.out_stride, active ? (uint32_t)a.d : 0u);
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      float v[VEC];
#pragma unroll
      for (int e = 0; e < VEC; ++e) v[e] = y[k][e] * qmul;
      store8<VEC>(pack_fp8<VEC>(v), ors, off8 + k * kStep8);
    }
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
