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
//  * Every finite input is served to the stated tolerance: a bf16 row whose
//    fp32 sum of squares underflows or overflows is detected after the
//    reduction and recomputed from the row scaled by 2^+-76 (exact), in a
//    branch the other rows skip.  (With a variance size below the row, y =
//    (r * factor) * w is formed in that order, and r * factor can pass
//    fp32's range where y would not; at the full size it is below
//    sqrt(hidden).)
//  * e4m3 codes come from the packed gfx950 v_cvt_pk_fp8_f32 (OCP format
//    on this target) after an explicit fmed3 clamp to +-448.
//  * x and out may alias: every element is loaded before the reduction and
//    stored after it by the same lane, so nothing is marked __restrict__.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

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
  __shared__ float red_scaled[WPR * RPB];  // rescaled sums (rows out of fp32 range)
  __shared__ float red_wide[WPR * RPB];    // dynamic e4m3: rescaled maxima

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
    if constexpr (kStatic) {
      qmul = 1.0f / *a.scale;
      // Keep the divide here, beside the loads, rather than after the row
      // reduction where it would lengthen each row's critical path.
      asm volatile("" ::"v"(qmul));
    }

    // 2. r = x + residual in fp32, rounded to 16 bits and stored back;
    //    sum of squares of the rounded r over the first var_cols channels
    //    (all of them unless the variance size is overridden), and max |r*w|
    //    for dynamic FP8.  Zero-filled vectors add nothing and their stores
    //    are dropped.
    if constexpr (kRes) {
#pragma unroll
      for (int k = 0; k < NV; ++k) {
        if constexpr (DT == kFP16) {
          xr[k] = add_f16<VEC>(xr[k], rr[k]);  // = fp32 add rounded to fp16, two per op
        } else {
          float f[VEC];
#pragma unroll
          for (int e = 0; e < VEC; ++e) f[e] = elem<DT, VEC>(xr[k], e) + elem<DT, VEC>(rr[k], e);
          xr[k] = pack<DT, VEC>(f);
        }
        store16<VEC>(xr[k], rrs, off16 + k * kStep16);
      }
    }
    // fma(a, b, nz) is a * b; with an fp16 operand it reads the half directly.
    const float nz = opaque_neg_zero();
    float ss = 0.0f;
    float mx = 0.0f;
    if (a.var_cols == a.hidden) {
#pragma unroll
      for (int k = 0; k < NV; ++k) ss = sum_squares<DT, VEC>(xr[k], ss);
    } else {
#pragma unroll
      for (int k = 0; k < NV; ++k) {
        const int col0 = (t + k * kTPR) * VEC;
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          // (Selected before squaring: an infinite channel past the variance
          // size must add nothing, and inf * 0 would add a NaN.)
          const float rf = col0 + e < a.var_cols ? elem<DT, VEC>(xr[k], e) : 0.0f;
          ss = __builtin_fmaf(rf, rf, ss);
        }
      }
    }
    // Dynamic e4m3: max |p| over the products p = r * w.  For 16-bit r and w
    // each product is exact in fp32 unless it leaves fp32's range (|p| >=
    // 2^128, or below 2^-126 with low bits lost).
    if constexpr (kDynamic) {
#pragma unroll
      for (int k = 0; k < NV; ++k) {
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          mx = fmaxf(mx, fabsf(__builtin_fmaf(elem<DT, VEC>(xr[k], e), elem<DT, VEC>(wr[k], e), nz)));
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
    float inv = rsqrtf(__builtin_fmaf(ss, a.inv_var, a.eps));
    float rmul = 1.0f;  // rescued rows: y = ((r * rmul) * inv) * w

    // 3b. Rows outside fp32's range.  A bf16 row whose squares underflow
    //     (every |r| below about 2^-75, with eps as small) or whose sum of
    //     squares overflows (|r| near bf16's largest values) gets its sum of
    //     squares again from r * 2^76 or r * 2^-76 -- powers of two, so the
    //     scaled values are exact -- and y = r * (2^+-76 / sqrt(ms 2^+-152
    //     + eps 2^+-152)) * w, the same quantity, with no intermediate out
    //     of range unless r times the true factor is.  Other rows never enter this branch, so their results are
    //     the plain formula's, bit for bit.  The branch is uniform over every
    //     row that shares a barrier: with several multi-wave rows per block,
    //     all of them enter when one needs it (their own rescaled sums are
    //     then unused).
    const float total = __builtin_fmaf(ss, a.inv_var, a.eps);
    const bool rescue = !(total >= 0x1p-96f) || !(ss <= 3.4028234e38f);
    bool enter = rescue;
    if constexpr (WPR > 1 && RPB > 1) {
      enter = false;
#pragma unroll
      for (int rr = 0; rr < RPB; ++rr) {
        float s = 0.0f;
#pragma unroll
        for (int i = 0; i < WPR; ++i) s += red_sum[rr * WPR + i];
        const float tt = __builtin_fmaf(s, a.inv_var, a.eps);
        enter = enter || !(tt >= 0x1p-96f) || !(s <= 3.4028234e38f);
      }
    }
    if (enter) {
      const float sc = ss < 1.0f ? 0x1p76f : 0x1p-76f;
      float s2 = 0.0f;
#pragma unroll
      for (int k = 0; k < NV; ++k) {
        // The packed row passes through an empty asm the compiler cannot
        // see through, so no unpacked copy of it is kept live across this
        // branch for the output step.
        asm volatile("" : "+v"(xr[k]));
        const int col0 = (t + k * kTPR) * VEC;
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          // Channels past the variance size are dropped before the scaling:
          // scaled by 2^76 they could overflow, and inf * 0 is NaN.
          const float rf = (col0 + e < a.var_cols ? elem<DT, VEC>(xr[k], e) : 0.0f) * sc;
          s2 = __builtin_fmaf(rf, rf, s2);
        }
      }
      s2 = wave_sum(s2);
      if constexpr (WPR > 1) {
        if (lane == 0) red_scaled[wave] = s2;
        __syncthreads();
        s2 = 0.0f;
#pragma unroll
        for (int i = 0; i < WPR; ++i) s2 += red_scaled[rib * WPR + i];
      }
      if (rescue) {
        // The true row factor is is * sc, exact while it is a normal fp32
        // number; then the row takes the plain order (r * factor) * w.  Only
        // a factor outside the normal range keeps the scaled operand,
        // ((r * sc) * is) * w.  (With a variance size below the row the other
        // channels can be far larger than the ones the mean runs over, and
        // r * 2^76 would overflow where r * factor does not.)
        const float is = rsqrtf(__builtin_fmaf(s2, a.inv_var, a.eps * sc * sc));
        const float g = is * sc;
        const bool normal = __float_as_uint(g) - 0x00800000u <= 0x7F7FFFFFu - 0x00800000u;
        rmul = normal ? g : sc;
        inv = normal ? 1.0f : is;
      }
    }

    // 4. y = r * inv * w, stored as 16 bits or as e4m3 codes.
    if constexpr (kDynamic) {
      // code = e4m3(y / scale) with scale = max|y| / 448.  Since y = p * inv
      // * rmul with one positive factor for the whole row, y / scale =
      // p * 448 / max|p|: the codes need the products and their max only.
      // That holds in fp32 while max|p| lies in [2^-96, 2^128): then 448 /
      // max|p| is finite and a product that lost low bits below 2^-126 is
      // off by less than 2^-54 of the max.  A row outside that range ("wide":
      // a product overflowed, or every product is below 2^-96 or zero) forms
      // its products from operands scaled by f = 2^-64 each (overflow) or
      // 2^64 each (tiny; an operand that would pass fp32's largest value is
      // held there, which only happens when the other one is zero):
      //  * down: the largest product's operands are >= 1, so they and it
      //    stay exact, the max is >= 1, and what smaller operands lose in
      //    scaling is below 2^-86 of it;
      //  * up: every operand stays exact and so does every product (at
      //    most 22 significant bits, none below 2^-138), and a max still
      //    below 2^-96 (products under 2^-224) is lifted by 2^100 more
      //    before 448 / max is formed.
      // The scale is formed in fp64 from the max and the factors, so it is
      // the rounded quotient whatever its magnitude.
      // (mx >= 0, so its bits order like its value: one subtract and one
      // unsigned compare test 2^-96 <= mx <= fp32's largest value.)
      const bool wide = __float_as_uint(mx) - 0x0F800000u > 0x7F7FFFFFu - 0x0F800000u;
      const float f = wide ? (mx > 1.0f ? 0x1p-64f : 0x1p64f) : 1.0f;
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
      // scaled product of one element (wide rows)
      auto pscaled = [&](int k, int e) {
        const float xs = __builtin_amdgcn_fmed3f(elem<DT, VEC>(xr[k], e) * f, -3.4028234e38f,
                                                 3.4028234e38f);
        const float ws = __builtin_amdgcn_fmed3f(elem<DT, VEC>(wr[k], e) * f, -3.4028234e38f,
                                                 3.4028234e38f);
        return xs * ws;
      };
      float m = mx;
      if (enter_w) {
        float m2 = 0.0f;
#pragma unroll
        for (int k = 0; k < NV; ++k) {
          asm volatile("" : "+v"(xr[k]), "+v"(wr[k]));
#pragma unroll
          for (int e = 0; e < VEC; ++e) m2 = fmaxf(m2, fabsf(pscaled(k, e)));
        }
        m2 = wave_max(m2);
        if constexpr (WPR > 1) {
          if (lane == 0) red_wide[wave] = m2;
          __syncthreads();
          m2 = 0.0f;
#pragma unroll
          for (int i = 0; i < WPR; ++i) m2 = fmaxf(m2, red_wide[rib * WPR + i]);
        }
        if (wide) m = m2;
      }
      // code = e4m3(y / s) = e4m3(formed product * lift * c).  The usual row
      // (products in range, no rescaling, max|y| = m * inv well inside
      // fp32) takes s = (m * inv) / 448 and c = 448 / m in fp32 (a multiply
      // by 1/448 and a hardware reciprocal, each within an ulp or two), the
      // scale written by one lane.  Any other row forms s in fp64: products as
      // formed are p / ung (ung = 1 / (f * f)), so s = m * ung * inv * rmul
      // / 448 with only exact powers of two besides the fp64 products,
      // rounded once to fp32.  While that s is a normal fp32 number it is
      // max|y| / 448 to within half an fp32 ulp and c = 448 / (lifted max);
      // otherwise the stored value is coarse or not finite and the codes
      // follow it: c = yscale / (s * lift / ung) in fp64 -- infinite when s
      // rounded to zero under a nonzero row, zero when it overflowed, as
      // y / s is.
      const float amax = m * inv;
      float c;
      float lift = 1.0f;  // a wide row's max below 2^-96 is lifted by 2^100
      // (amax >= 0 or NaN; NaN's bits lie above 2^100's.)
      if (!wide && !rescue && __float_as_uint(amax) - 0x0D800000u <= 0x71800000u - 0x0D800000u) {
        // m / 448 lies in [2^-105, 2^120), so its hardware reciprocal (1
        // ulp) is a normal number; the codes allow the fp32 roundings.
        if (active && t == 0) a.scale[row] = amax * (1.0f / 448.0f);
        c = __builtin_amdgcn_rcpf(m * (1.0f / 448.0f));
      } else {
        const double ung = f == 1.0f ? 1.0 : (f < 1.0f ? 0x1p128 : 0x1p-128);
        const double yscale = (double)inv * (double)rmul;  // y = p * yscale
        const float s = (float)((double)m * ung * yscale * (1.0 / 448.0));
        if (active && t == 0) a.scale[row] = s;
        if (m < 0x1p-96f) lift = 0x1p100f;
        if (s >= 0x1p-126f && s <= 3.4028234e38f) {
          c = 448.0f / (m * lift);
        } else {
          c = m > 0.0f ? (float)(yscale * ung / ((double)s * (double)lift)) : 0.0f;
        }
      }
      const __amdgpu_buffer_rsrc_t ors = row_rsrc(
          static_cast<uint8_t*>(a.out) + arow * a.out_stride, active ? row_bytes8 : 0u);
      if (wide) {
#pragma unroll
        for (int k = 0; k < NV; ++k) {
          // (Laundered so the scaled operands are formed again here rather
          // than kept live from the max loop.)
          asm volatile("" : "+v"(xr[k]), "+v"(wr[k]));
          float y[VEC];
#pragma unroll
          for (int e = 0; e < VEC; ++e) y[e] = (pscaled(k, e) * lift) * c;
          store8<VEC>(pack_fp8<VEC>(y), ors, off8 + k * kStep8);
        }
      } else {
#pragma unroll
        for (int k = 0; k < NV; ++k) {
          float y[VEC];
#pragma unroll
          for (int e = 0; e < VEC; ++e) {
            y[e] = __builtin_fmaf(elem<DT, VEC>(xr[k], e), elem<DT, VEC>(wr[k], e), nz) * c;
          }
          store8<VEC>(pack_fp8<VEC>(y), ors, off8 + k * kStep8);
        }
      }
      return;
    }

    // Static e4m3 multiplies by 1/s.  For fp16 rows the product r * w is
    // exact in fp32 (at most 22 significant bits, magnitude within
    // [2^-48, 2^32] or zero), so y / s = (r * w) * (inv / s) with the row
    // constant inv / s; held at fp32's largest value if it overflows, which
    // still saturates every nonzero product and keeps zeros zero.  bf16
    // products can leave fp32's range, so bf16 rows form y first.
    const float cq = kStatic ? fminf(inv * qmul, 3.4028234e38f) : 0.0f;

    // A rescaled row takes its own copy of the loop (y = ((r * rmul) * inv)
    // * w), so the other rows pay no extra multiply per element.
    auto emit = [&](auto scaled) {
      constexpr bool kScaled = decltype(scaled)::value;
      if constexpr (kFp8) {
        const __amdgpu_buffer_rsrc_t ors = row_rsrc(
            static_cast<uint8_t*>(a.out) + arow * a.out_stride, active ? row_bytes8 : 0u);
#pragma unroll
        for (int k = 0; k < NV; ++k) {
          float y[VEC];
#pragma unroll
          for (int e = 0; e < VEC; ++e) {
            if constexpr (kScaled) {
              y[e] = elem<DT, VEC>(xr[k], e) * rmul * inv * elem<DT, VEC>(wr[k], e) * qmul;
            } else if constexpr (DT == kFP16) {
              y[e] = __builtin_fmaf(elem<DT, VEC>(xr[k], e), elem<DT, VEC>(wr[k], e), nz) * cq;
            } else {
              const float t = __builtin_fmaf(elem<DT, VEC>(xr[k], e), inv, nz);
              y[e] = __builtin_fmaf(elem<DT, VEC>(wr[k], e), t, nz) * qmul;
            }
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
            if constexpr (kScaled) {
              y[e] = elem<DT, VEC>(xr[k], e) * rmul * inv * elem<DT, VEC>(wr[k], e);
            } else {
              const float t = __builtin_fmaf(elem<DT, VEC>(xr[k], e), inv, nz);
              y[e] = __builtin_fmaf(elem<DT, VEC>(wr[k], e), t, nz);
            }
          }
          store16<VEC>(pack<DT, VEC>(y), ors, off16 + k * kStep16);
        }
      }
    };
    if (rescue) {
      // (Laundered as above, so the two loops share no unpacked values that
      // the compiler would hoist above the branch and keep live.)
#pragma unroll
      for (int k = 0; k < NV; ++k) asm volatile("" : "+v"(xr[k]));
      emit(std::true_type{});
    } else {
      emit(std::false_type{});
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
