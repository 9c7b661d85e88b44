// arn_device.h -- device helpers shared by the gfx950 kernels: 16-bit and
// e4m3 conversions, bounded buffer loads/stores of row segments, and wave64
// reductions.  Included by the kernel units only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "arn_internal.h"

namespace arn {
namespace dev {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------------------
// 16-bit <-> fp32.  bf16 is the upper half of an fp32; fp16 converts with
// v_cvt_f32_f16.  fp32 -> 16-bit rounds to nearest even: v_cvt_pk_bf16_f32
// on gfx950 for bf16, v_cvt_f16_f32 for fp16 (never the round-toward-zero
// v_cvt_pkrtz_f16_f32).
// ---------------------------------------------------------------------------
template <int DT>
__device__ __forceinline__ float lo_f32(uint32_t w) {
  if constexpr (DT == kBF16) {
    return __uint_as_float(w << 16);
  } else {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xFFFFu));
  }
}

template <int DT>
__device__ __forceinline__ float hi_f32(uint32_t w) {
  if constexpr (DT == kBF16) {
    return __uint_as_float(w & 0xFFFF0000u);
  } else {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
  }
}

template <int DT>
__device__ __forceinline__ uint32_t pack2(float a, float b) {
  f32x2 v;
  v.x = a;
  v.y = b;
  if constexpr (DT == kBF16) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
  } else {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2));
  }
}

// VEC 16-bit elements as one memory access.
template <int VEC> struct RawT;
template <> struct RawT<8> { using type = u32x4; };
template <> struct RawT<4> { using type = u32x2; };
template <> struct RawT<2> { using type = uint32_t; };
template <> struct RawT<1> { using type = uint16_t; };
template <int VEC> using Raw = typename RawT<VEC>::type;

// VEC e4m3 codes as one memory access.
template <int VEC> struct Fp8RawT;
template <> struct Fp8RawT<8> { using type = u32x2; };
template <> struct Fp8RawT<4> { using type = uint32_t; };
template <> struct Fp8RawT<2> { using type = uint16_t; };
template <> struct Fp8RawT<1> { using type = uint8_t; };
template <int VEC> using Fp8Raw = typename Fp8RawT<VEC>::type;

template <int DT, int VEC>
__device__ __forceinline__ float elem(const Raw<VEC>& r, int e) {
  if constexpr (VEC == 1) {
    return lo_f32<DT>((uint32_t)r);
  } else if constexpr (VEC == 2) {
    return (e & 1) ? hi_f32<DT>(r) : lo_f32<DT>(r);
  } else {
    const uint32_t w = r[e >> 1];
    return (e & 1) ? hi_f32<DT>(w) : lo_f32<DT>(w);
  }
}

template <int DT, int VEC>
__device__ __forceinline__ Raw<VEC> pack(const float (&f)[VEC]) {
  if constexpr (VEC == 1) {
    return (uint16_t)(pack2<DT>(f[0], 0.0f) & 0xFFFFu);
  } else if constexpr (VEC == 2) {
    return pack2<DT>(f[0], f[1]);
  } else {
    Raw<VEC> r;
#pragma unroll
    for (int i = 0; i < VEC / 2; ++i) r[i] = pack2<DT>(f[2 * i], f[2 * i + 1]);
    return r;
  }
}

template <int DT, int VEC>
__device__ __forceinline__ Raw<VEC> ones() {
  constexpr uint32_t one = (DT == kBF16) ? 0x3F80u : 0x3C00u;
  if constexpr (VEC == 1) {
    return (uint16_t)one;
  } else if constexpr (VEC == 2) {
    return one | (one << 16);
  } else {
    Raw<VEC> r;
#pragma unroll
    for (int i = 0; i < VEC / 2; ++i) r[i] = one | (one << 16);
    return r;
  }
}

// ---------------------------------------------------------------------------
// Packed 16-bit arithmetic on whole 32-bit words (two elements each).
// ---------------------------------------------------------------------------
// The fp16 residual add as one packed fp16 add per word (v_pk_add_f16).  It
// equals the fp32 add of the two values rounded to fp16: fp32 carries at
// least 2 * 11 + 2 bits, so rounding the exact sum first to fp32 and then to
// fp16 gives the correctly rounded fp16 sum (double-rounding theorem), which
// is what the packed add returns.  (bf16 has no packed add on gfx950; its
// sum goes through fp32 and v_cvt_pk_bf16_f32.)
template <int VEC>
__device__ __forceinline__ Raw<VEC> add_f16(const Raw<VEC>& a, const Raw<VEC>& b) {
  if constexpr (VEC == 1) {
    return __builtin_bit_cast(uint16_t, (_Float16)(__builtin_bit_cast(_Float16, a) +
                                                    __builtin_bit_cast(_Float16, b)));
  } else if constexpr (VEC == 2) {
    return __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, a) + __builtin_bit_cast(f16x2, b));
  } else {
    Raw<VEC> r;
#pragma unroll
    for (int i = 0; i < VEC / 2; ++i) {
      // Each element is copied to a plain word first: clang's
      // __builtin_bit_cast of an ext-vector element expression (a[i])
      // reads element 0 whatever i is.
      const uint32_t ai = a[i], bi = b[i];
      r[i] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, ai) + __builtin_bit_cast(f16x2, bi));
    }
    return r;
  }
}

// acc + the squares of the two 16-bit values of a word, with one
// v_dot2_f32_{f16,bf16}: the products are exact in fp32, the sums fp32.
template <int DT>
__device__ __forceinline__ float dot2_self(uint32_t w, float acc) {
  if constexpr (DT == kBF16) {
    const bf16x2 v = __builtin_bit_cast(bf16x2, w);
    return __builtin_amdgcn_fdot2_f32_bf16(v, v, acc, false);
  } else {
    const f16x2 v = __builtin_bit_cast(f16x2, w);
    return __builtin_amdgcn_fdot2(v, v, acc, false);
  }
}

// acc + the sum of squares of the VEC values of one vector.
template <int DT, int VEC>
__device__ __forceinline__ float sum_squares(const Raw<VEC>& r, float acc) {
  if constexpr (VEC == 1) {
    const float f = lo_f32<DT>((uint32_t)r);
    return __builtin_fmaf(f, f, acc);
  } else if constexpr (VEC == 2) {
    return dot2_self<DT>(r, acc);
  } else {
#pragma unroll
    for (int i = 0; i < VEC / 2; ++i) {
      const uint32_t w = r[i];
      acc = dot2_self<DT>(w, acc);
    }
    return acc;
  }
}

// A -0.0f the compiler cannot see through.  fma(a, b, -0) is a * b exactly
// (signed zeros included), and with an fp16 operand and an addend the
// compiler does not know it selects v_fma_mix_f32, which reads the fp16 half
// of a register directly instead of converting it first.
__device__ __forceinline__ float opaque_neg_zero() {
  float z = -0.0f;
  asm volatile("" : "+v"(z));
  return z;
}

// ---------------------------------------------------------------------------
// OCP e4m3: clamp to the finite range, then the packed gfx950 convert
// (round to nearest even).  word_sel picks which 16-bit half of the
// destination dword receives the two codes.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float sat448(float v) {
  return __builtin_amdgcn_fmed3f(v, -448.0f, 448.0f);
}

__device__ __forceinline__ uint32_t fp8x4(float a, float b, float c, float d) {
  // The first convert writes the low 16 bits and keeps the high 16 of its
  // third operand, which the second convert then overwrites: any value
  // already in a register serves (a literal 0 would cost a move).
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(sat448(a), sat448(b), __float_as_int(a), false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(sat448(c), sat448(d), w, true);
  return (uint32_t)w;
}

template <int VEC>
__device__ __forceinline__ Fp8Raw<VEC> pack_fp8(const float (&f)[VEC]) {
  if constexpr (VEC == 8) {
    u32x2 r;
    r.x = fp8x4(f[0], f[1], f[2], f[3]);
    r.y = fp8x4(f[4], f[5], f[6], f[7]);
    return r;
  } else if constexpr (VEC == 4) {
    return fp8x4(f[0], f[1], f[2], f[3]);
  } else if constexpr (VEC == 2) {
    return (uint16_t)(__builtin_amdgcn_cvt_pk_fp8_f32(sat448(f[0]), sat448(f[1]), 0, false) &
                      0xFFFF);
  } else {
    return (uint8_t)(__builtin_amdgcn_cvt_pk_fp8_f32(sat448(f[0]), sat448(f[0]), 0, false) &
                     0xFF);
  }
}

// ---------------------------------------------------------------------------
// Wave64 reductions: four DPP steps give every lane its 16-lane row total
// (xor 1, xor 2, half-row mirror, row mirror), then the four row totals are
// read with v_readlane and combined in a fixed order.
// ---------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}

__device__ __forceinline__ float lane_f(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

constexpr int kDppXor1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppMirror = 0x140;

__device__ __forceinline__ float wave_sum(float v) {
  v += dpp<kDppXor1>(v);
  v += dpp<kDppXor2>(v);
  v += dpp<kDppHalfMirror>(v);
  v += dpp<kDppMirror>(v);
  return (lane_f(v, 0) + lane_f(v, 16)) + (lane_f(v, 32) + lane_f(v, 48));
}

__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp<kDppXor1>(v));
  v = fmaxf(v, dpp<kDppXor2>(v));
  v = fmaxf(v, dpp<kDppHalfMirror>(v));
  v = fmaxf(v, dpp<kDppMirror>(v));
  return fmaxf(fmaxf(lane_f(v, 0), lane_f(v, 16)), fmaxf(lane_f(v, 32), lane_f(v, 48)));
}

// Max over the wave in fp64 (lane permutes; for rows whose values leave
// fp32's range, so not on the hot path).  Every lane gets the result.
__device__ __forceinline__ double wave_max_f64(double v) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) v = fmax(v, __shfl_xor(v, m));
  return v;
}

// ---------------------------------------------------------------------------
// Row accesses go through buffer instructions: a descriptor in SGPRs holds
// the row's base address and its length in bytes (num_records), and each
// lane supplies a 32-bit byte offset.  An access at or beyond num_records
// reads zeros and drops stores, so the ragged end of a row needs no
// branches, a row past the last one (num_records = 0) touches nothing, and
// no access can leave its own row.  Word 3 is the gfx9 raw-buffer format
// (DATA_FORMAT = 32 bit).
// ---------------------------------------------------------------------------
constexpr int kRsrcWord3 = 0x00020000;

// Cache policy of the memory instructions.  x, residual and out are each
// touched once per call, so they stream with the non-temporal hint (nt);
// the weight, read by every row, stays cacheable.
constexpr int kCacheDefault = 0;
constexpr int kCacheStream = 2;  // nt

__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           kRsrcWord3);
}

template <int VEC, int CP>
__device__ __forceinline__ Raw<VEC> load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  if constexpr (VEC == 8) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, CP);
  } else if constexpr (VEC == 4) {
    return __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, CP);
  } else if constexpr (VEC == 2) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, CP);
  } else {
    return __builtin_amdgcn_raw_buffer_load_b16(r, (int)off, 0, CP);
  }
}

template <int VEC>
__device__ __forceinline__ void store16(Raw<VEC> v, __amdgpu_buffer_rsrc_t r, uint32_t off) {
  if constexpr (VEC == 8) {
    __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)off, 0, kCacheStream);
  } else if constexpr (VEC == 4) {
    __builtin_amdgcn_raw_buffer_store_b64(v, r, (int)off, 0, kCacheStream);
  } else if constexpr (VEC == 2) {
    __builtin_amdgcn_raw_buffer_store_b32(v, r, (int)off, 0, kCacheStream);
  } else {
    __builtin_amdgcn_raw_buffer_store_b16(v, r, (int)off, 0, kCacheStream);
  }
}

template <int VEC>
__device__ __forceinline__ void store8(Fp8Raw<VEC> v, __amdgpu_buffer_rsrc_t r, uint32_t off) {
  if constexpr (VEC == 8) {
    __builtin_amdgcn_raw_buffer_store_b64(v, r, (int)off, 0, kCacheStream);
  } else if constexpr (VEC == 4) {
    __builtin_amdgcn_raw_buffer_store_b32(v, r, (int)off, 0, kCacheStream);
  } else if constexpr (VEC == 2) {
    __builtin_amdgcn_raw_buffer_store_b16(v, r, (int)off, 0, kCacheStream);
  } else {
    __builtin_amdgcn_raw_buffer_store_b8(v, r, (int)off, 0, kCacheStream);
  }
}

}  // namespace dev
}  // namespace arn
