// Internal interface between the host dispatcher (arn_api.hip) and the
// e4m3 GEMM unit (arn_gemm.hip, compiled once per output dtype).  Kept apart
// from arn_internal.h so that the norm and SwiGLU kernels do not depend on it.
#pragma once

#include <stdint.h>

namespace arn {

// e4m3 GEMM arguments: C[m][n] = sa(m) sb(n) sum_k A[m][k] B[n][k].
struct GemmArgs {
  void* c;             // m x n of the 16-bit output dtype, row stride ldc elements
  int64_t ldc;
  const void* a;       // m x k codes, row stride lda bytes
  int64_t lda;
  const float* scale_a;
  const void* b;       // n x k codes, row stride ldb bytes
  int64_t ldb;
  const float* scale_b;
  int64_t m;
  int64_t n;
  int64_t k;
  int32_t a_per_row;
  int32_t b_per_row;
  // Split K across gridDim.y blocks per column tile (1: no split).  Each
  // split covers k steps [y * steps_per_split, (y + 1) * steps_per_split);
  // partial tiles go to `partial` (tile-major, splits inner) and the block
  // that finishes a tile last (counted in `counters`, one per column tile,
  // zero on entry and left zero) sums them in split order.
  int32_t splits;
  int32_t steps_per_split;
  float* partial;
  int32_t* counters;
};

// One compiled GEMM shape: MT x NT tiles of 16 x 16 outputs per block, K
// split over `waves` waves.
struct GemmCfg {
  int mt;
  int nt;
  int waves;
  const void* fn;      // row-major weight
  const void* fn_pre;  // pre-shuffled weight
};

// Weight pre-shuffle into MFMA tile order (see arn_gemm.hip).
struct PreshuffleArgs {
  void* dst;
  const void* src;
  int64_t ldb;
  int64_t n;
  int64_t k;
  int64_t ntiles;       // ceil(n / 16)
  int64_t nsteps;       // ceil(k / 128)
  int64_t panel_tiles;  // column tiles per panel (panel_tiles_for(nsteps))
  int aligned;          // src and ldb are multiples of 16 bytes
};

// The pre-shuffled weight is a sequence of panels of `panel_tiles` column
// tiles (the last one may hold fewer); inside a panel the 2 KiB MFMA tiles
// are stored k-step major: all of the panel's tiles for step 0, then step 1,
// and so on.  A panel is at most 1 GiB, so every offset a GEMM launch uses
// fits the 32-bit buffer offsets, and the tile count is a multiple of 4 so
// that no column group of a GEMM block straddles two panels.
inline int64_t panel_tiles_for(int64_t nsteps) {
  const int64_t t = (int64_t(1) << 30) / (nsteps * 2048) / 4 * 4;
  return t < 4 ? 4 : t;
}

struct GemmTable {
  const GemmCfg* cfgs;
  int count;
};

}  // namespace arn

#define ARN_GEMM_TABLE_NAME_(DT) arn_gemm_cfgs_d##DT
#define ARN_GEMM_TABLE_NAME(DT) ARN_GEMM_TABLE_NAME_(DT)
extern const arn::GemmTable ARN_GEMM_TABLE_NAME(0);
extern const arn::GemmTable ARN_GEMM_TABLE_NAME(1);
extern const void* const arn_preshuffle_fn;
