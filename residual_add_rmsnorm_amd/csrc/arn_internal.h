// Internal interface between the host dispatcher (arn_api.hip) and the
// row-kernel instantiation units (arn_kernels.hip, compiled once per
// operator kind and dtype; arn_glu.hip, once per SwiGLU output mode and
// dtype).  The GEMM's interface is arn_gemm.h.
#pragma once

#include <stdint.h>

namespace arn {

// Operator kind: bit 0 = residual add, bit 1 = static e4m3 out,
// bit 2 = dynamic e4m3 out.  Kinds without bit 1/2 write 16-bit y.
enum Kind : int {
  kPlain = 0,
  kFused = 1,
  kPlainFp8Static = 2,
  kFusedFp8Static = 3,
  kPlainFp8Dynamic = 4,
  kFusedFp8Dynamic = 5,
  kNumKinds = 6,
};

enum Dtype : int { kBF16 = 0, kFP16 = 1, kNumDtypes = 2 };

// Largest number of partial inputs of the all-reduce form.
constexpr int kMaxParts = 8;

// Kernel arguments, passed by value.  Strides are in elements of each
// tensor; `out` holds 16-bit elements or e4m3 bytes depending on the kind.
struct Args {
  void* out;
  int64_t out_stride;
  const void* x;
  int64_t x_stride;
  void* res;
  int64_t res_stride;
  const void* w;      // nullptr: w = 1
  float* scale;       // static: 1 value read; dynamic: `rows` values written
  int64_t rows;
  int32_t hidden;
  int32_t var_cols;   // channels in the mean of squares (== hidden unless overridden)
  float eps;
  float inv_var;      // 1.0f / var_cols
  // All-reduce form only (kernels built with ARN_SUM=1): x is the fp32
  // rank-order sum of the nparts parts (row stride x_stride), rounded once
  // to 16 bits.
  const void* parts[kMaxParts];
  int32_t nparts;
};

// SwiGLU output modes.
enum GluMode : int { kGluPlain = 0, kGluStatic = 1, kGluDynamic = 2, kNumGluModes = 3 };

// SwiGLU kernel arguments: out = silu(gate) * up over `d` columns per row.
struct GluArgs {
  void* out;
  int64_t out_stride;
  const void* gate;
  int64_t gate_stride;
  const void* up;
  int64_t up_stride;
  float* scale;  // static: 1 value read; dynamic: `rows` values written
  int64_t rows;
  int32_t d;
};

// One compiled kernel shape.  A lane owns vectors of VEC contiguous
// elements; WPR waves (64 lanes each) share a row; a lane keeps up to NV
// vectors of its row in registers; a block holds RPB rows.
struct Tile {
  int vec;
  int wpr;
  int nv;
  int rpb;
  const void* fn;  // host handle of the __global__ function
};

struct TileTable {
  const Tile* tiles;
  int count;
};

}  // namespace arn

// Defined by each instantiation unit.
#define ARN_TABLE_NAME_(KIND, DT) arn_tiles_k##KIND##_d##DT
#define ARN_TABLE_NAME(KIND, DT) ARN_TABLE_NAME_(KIND, DT)
#define ARN_DECLARE_TABLE(KIND, DT) extern const arn::TileTable ARN_TABLE_NAME(KIND, DT);

ARN_DECLARE_TABLE(0, 0)
ARN_DECLARE_TABLE(0, 1)
ARN_DECLARE_TABLE(1, 0)
ARN_DECLARE_TABLE(1, 1)
ARN_DECLARE_TABLE(2, 0)
ARN_DECLARE_TABLE(2, 1)
ARN_DECLARE_TABLE(3, 0)
ARN_DECLARE_TABLE(3, 1)
ARN_DECLARE_TABLE(4, 0)
ARN_DECLARE_TABLE(4, 1)
ARN_DECLARE_TABLE(5, 0)
ARN_DECLARE_TABLE(5, 1)

#define ARN_SUM_TABLE_NAME_(KIND, DT) arn_sum_tiles_k##KIND##_d##DT
#define ARN_SUM_TABLE_NAME(KIND, DT) ARN_SUM_TABLE_NAME_(KIND, DT)
#define ARN_DECLARE_SUM_TABLE(KIND, DT) extern const arn::TileTable ARN_SUM_TABLE_NAME(KIND, DT);

ARN_DECLARE_SUM_TABLE(0, 0)
ARN_DECLARE_SUM_TABLE(0, 1)
ARN_DECLARE_SUM_TABLE(1, 0)
ARN_DECLARE_SUM_TABLE(1, 1)
ARN_DECLARE_SUM_TABLE(2, 0)
ARN_DECLARE_SUM_TABLE(2, 1)
ARN_DECLARE_SUM_TABLE(3, 0)
ARN_DECLARE_SUM_TABLE(3, 1)
ARN_DECLARE_SUM_TABLE(4, 0)
ARN_DECLARE_SUM_TABLE(4, 1)
ARN_DECLARE_SUM_TABLE(5, 0)
ARN_DECLARE_SUM_TABLE(5, 1)

#define ARN_GLU_TABLE_NAME_(MODE, DT) arn_glu_tiles_m##MODE##_d##DT
#define ARN_GLU_TABLE_NAME(MODE, DT) ARN_GLU_TABLE_NAME_(MODE, DT)
#define ARN_DECLARE_GLU_TABLE(MODE, DT) extern const arn::TileTable ARN_GLU_TABLE_NAME(MODE, DT);

ARN_DECLARE_GLU_TABLE(0, 0)
ARN_DECLARE_GLU_TABLE(0, 1)
ARN_DECLARE_GLU_TABLE(1, 0)
ARN_DECLARE_GLU_TABLE(1, 1)
ARN_DECLARE_GLU_TABLE(2, 0)
ARN_DECLARE_GLU_TABLE(2, 1)
