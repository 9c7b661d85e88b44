// arn_api.hip -- the C ABI declared in include/arn.h: argument checks, the
// choice of kernel shape, and the launch, for the norm, SwiGLU and GEMM
// kernels.  Host code only.
//
// Norm argument rules follow the vLLM API page "vllm.kernels.aiter_ops"
// (rms_add_no_var_16bit_only, rms_no_var_16bit_only, flatten_to_2d_is_free):
// 16-bit activations, a weight of the same dtype or none, unit element
// stride; the named entry points take no variance-size override (arn_norm
// adds one).  Anything else is refused before any HIP call, and nothing is
// ever copied to make an input acceptable.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "arn.h"
#include "arn_tuning.h"
#include "arn_internal.h"
#include "arn_gemm.h"

namespace {

using arn::Args;
using arn::GemmArgs;
using arn::GemmCfg;
using arn::GemmTable;
using arn::panel_tiles_for;
using arn::Tile;
using arn::TileTable;

const TileTable* table_for(int kind, int dtype) {
  static const TileTable* const tables[arn::kNumKinds][arn::kNumDtypes] = {
      {&ARN_TABLE_NAME(0, 0), &ARN_TABLE_NAME(0, 1)},
      {&ARN_TABLE_NAME(1, 0), &ARN_TABLE_NAME(1, 1)},
      {&ARN_TABLE_NAME(2, 0), &ARN_TABLE_NAME(2, 1)},
      {&ARN_TABLE_NAME(3, 0), &ARN_TABLE_NAME(3, 1)},
      {&ARN_TABLE_NAME(4, 0), &ARN_TABLE_NAME(4, 1)},
      {&ARN_TABLE_NAME(5, 0), &ARN_TABLE_NAME(5, 1)},
  };
  return tables[kind][dtype];
}

const TileTable* sum_table_for(int kind, int dtype) {
  static const TileTable* const tables[arn::kNumKinds][arn::kNumDtypes] = {
      {&ARN_SUM_TABLE_NAME(0, 0), &ARN_SUM_TABLE_NAME(0, 1)},
      {&ARN_SUM_TABLE_NAME(1, 0), &ARN_SUM_TABLE_NAME(1, 1)},
      {&ARN_SUM_TABLE_NAME(2, 0), &ARN_SUM_TABLE_NAME(2, 1)},
      {&ARN_SUM_TABLE_NAME(3, 0), &ARN_SUM_TABLE_NAME(3, 1)},
      {&ARN_SUM_TABLE_NAME(4, 0), &ARN_SUM_TABLE_NAME(4, 1)},
      {&ARN_SUM_TABLE_NAME(5, 0), &ARN_SUM_TABLE_NAME(5, 1)},
  };
  return tables[kind][dtype];
}

const TileTable* glu_table_for(int mode, int dtype) {
  static const TileTable* const tables[arn::kNumGluModes][arn::kNumDtypes] = {
      {&ARN_GLU_TABLE_NAME(0, 0), &ARN_GLU_TABLE_NAME(0, 1)},
      {&ARN_GLU_TABLE_NAME(1, 0), &ARN_GLU_TABLE_NAME(1, 1)},
      {&ARN_GLU_TABLE_NAME(2, 0), &ARN_GLU_TABLE_NAME(2, 1)},
  };
  return tables[mode][dtype];
}

const char* const kGluNames[arn::kNumGluModes] = {"silu_mul", "silu_mul_fp8s", "silu_mul_fp8d"};

const char* const kKindNames[arn::kNumKinds] = {"plain",      "fused_add",      "plain_fp8s",
                                                "fused_add_fp8s", "plain_fp8d", "fused_add_fp8d"};

// Settings of the tuning aids (arn_tuning.h), one copy per calling
// thread, so that forcing a shape on one thread never changes or refuses
// another thread's calls.
// Forced tile (arn_set_tile); 0 = automatic.  Packed as wpr << 8 | nv.
thread_local int g_forced_tile = 0;

thread_local char g_last_plan[160] = "";
thread_local int g_last_plan_len = 0;

// Compute units of the current device, cached per device.
int cu_count() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int v = cache[dev].load(std::memory_order_relaxed);
  if (v > 0) return v;
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0) {
    cus = 256;
  }
  cache[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

struct Request {
  int kind;
  int dtype;
  void* out;
  int64_t out_stride;
  const void* x;
  int64_t x_stride;
  void* res;
  int64_t res_stride;
  const void* w;
  float* scale;
  float eps;
  int64_t rows;
  int64_t hidden;
  hipStream_t stream;
  int64_t var_cols = 0;  // 0: hidden
  // All-reduce form: x is the rank-order sum of nparts parts (x unused).
  const void* const* parts = nullptr;
  int nparts = 0;
};

bool aligned(const void* p, uintptr_t bytes) {
  return (reinterpret_cast<uintptr_t>(p) % bytes) == 0;
}

// Widest access (in 16-bit elements) that every row start and the row
// length allow.
int choose_vec(const Request& r) {
  const bool fp8 = (r.kind & 6) != 0;
  for (int vec = 8; vec > 1; vec /= 2) {
    const uintptr_t b16 = 2u * vec;
    bool ok = r.hidden % vec == 0 && r.x_stride % vec == 0 && aligned(r.x, b16);
    for (int g = 0; g < r.nparts; ++g) ok = ok && aligned(r.parts[g], b16);
    if (r.res) ok = ok && r.res_stride % vec == 0 && aligned(r.res, b16);
    if (r.w) ok = ok && aligned(r.w, b16);
    if (fp8) {
      ok = ok && r.out_stride % vec == 0 && aligned(r.out, vec);
    } else {
      ok = ok && r.out_stride % vec == 0 && aligned(r.out, b16);
    }
    if (ok) return vec;
  }
  return 1;
}

int pow2_ceil(int64_t v) {
  int p = 1;
  while (p < v && p < (1 << 20)) p *= 2;
  return p;
}

// Kernel shape.  A row is split over `wpr` waves so that each lane holds
// only a few vectors.  Measured on MI355X:
//  * fused kinds, many rows (at least 4 per CU): rows of eight waves
//    (512-thread blocks), at most two 128-bit vectors per lane (about 40
//    VGPRs, eight waves per SIMD); one-wave rows holding a whole 8192-wide
//    row run 20-25% slower.
//  * compact tiles (`compact_nv` > 0), many rows: the fewest waves, at most
//    four, whose lanes hold at most two vectors, then up to `compact_nv`
//    vectors per lane.  Kinds that move few bytes per element or carry a
//    large fixed cost per row (barrier, reductions, scale store) gain from
//    more rows per CU and fewer idle lane slots: the plain kinds (up to
//    four vectors: 65536 rows of dynamic e4m3 2048-6144 wide take 14-41%
//    less time than with eight-wave rows), SwiGLU (d <= 4096: 22-31%), the
//    fused dynamic-e4m3 kind (1536-3584 wide: 5-21%) and the all-reduce
//    form over two or three parts (4096 wide: 7-8%), up to two vectors.
//    Rows too wide for that take the rule above.
//  * few rows (decode): eight waves per row, up to four vectors per lane,
//    finish each row soonest.
//  * `waves` > 0 (fused kinds on 128-bit accesses, rows 4097-8192 elements
//    wide, at most two rows per CU: decode batches up to twice the CU
//    count): rows of that many waves.  Measured against eight-wave
//    rows at 5120, 7168 and 8192 wide, 16-bit, static and dynamic e4m3,
//    fp16 and bf16, on 256 CUs:
//      - up to 1.25 rows per CU, four waves: at 256 rows 0.1-15% less time
//        in every case; over 160-320 rows up to 7% less for fp16 and
//        within +-3.3% for bf16;
//      - at most half a row per CU, four waves for fp16 rows only (1-128
//        rows: 2.9% less time over 54 cases, -8.8% to +1.5%); bf16 rows,
//        whose add has no packed form and so more VALU work per element,
//        ran up to 5% slower with four waves there and keep eight;
//      - 1.25 to 2 rows per CU, two waves with eight vectors per lane when
//        that covers the row with little idle (more than 768 vectors, i.e.
//        7168-8192 wide): 0.2-20% less time in all 36 cases of 384-512
//        rows (from 2.5 rows per CU on it loses 3-22%); narrower rows keep
//        four waves there (5120 wide: -5% to +1.7%).
// Among the compiled tiles of the chosen wave count, the one with the
// fewest per-lane vectors that covers the row (and at least `min_nv`) is
// taken; failing that, any tile that covers the row.
const Tile* choose_tile(const TileTable* table, int vec, int64_t nvec, int64_t rows, int cus,
                        bool lean = false, int compact_nv = 0, int waves = 0) {
  const int forced = g_forced_tile;
  if (forced != 0) {
    const int fw = forced >> 8, fn = forced & 0xFF;
    for (int i = 0; i < table->count; ++i) {
      const Tile& t = table->tiles[i];
      if (t.vec == vec && t.wpr == fw && t.nv == fn) {
        return (int64_t)64 * t.wpr * t.nv >= nvec ? &t : nullptr;
      }
    }
    return nullptr;
  }
  const bool many_rows = rows >= (int64_t)4 * cus;
  if (waves > 0) {
    const int64_t per_lane = (nvec + 64 * waves - 1) / (64 * waves);
    const Tile* pick = nullptr;
    for (int i = 0; i < table->count; ++i) {
      const Tile& t = table->tiles[i];
      if (t.vec == vec && t.wpr == waves && t.nv >= per_lane && (!pick || t.nv < pick->nv)) {
        pick = &t;
      }
    }
    if (pick) return pick;
  }
  if (compact_nv > 0 && many_rows) {
    int w = 4;
    while (w > 1 && (int64_t)64 * (w / 2) * 2 >= nvec) w /= 2;
    const int64_t per_lane = (nvec + 64 * w - 1) / (64 * w);
    const Tile* pick = nullptr;
    for (int i = 0; per_lane <= compact_nv && i < table->count; ++i) {
      const Tile& t = table->tiles[i];
      if (t.vec == vec && t.wpr == w && t.nv >= per_lane && t.nv <= compact_nv &&
          (!pick || t.nv < pick->nv)) {
        pick = &t;
      }
    }
    if (pick) return pick;
  }
  // lean: each vector brings several inputs (the all-reduce form), so one
  // vector per lane with more waves per row streams best.
  const int64_t target_nv = lean ? 1 : (many_rows ? 2 : 4);
  const int64_t min_nv = lean || !many_rows ? 1 : 2;
  const int wpr_floor = 8;
  int wpr = pow2_ceil((nvec + 64 * target_nv - 1) / (64 * target_nv));
  const int need1 = pow2_ceil((nvec + 63) / 64);  // waves if each lane held one vector
  if (wpr < wpr_floor) wpr = need1 < wpr_floor ? need1 : wpr_floor;
  if (wpr > 16) wpr = 16;

  const Tile* best = nullptr;
  for (int w = wpr; w <= 16 && !best; w *= 2) {
    int64_t per_lane = (nvec + 64 * w - 1) / (64 * w);
    if (per_lane < min_nv) per_lane = min_nv;
    for (int i = 0; i < table->count; ++i) {
      const Tile& t = table->tiles[i];
      if (t.vec == vec && t.wpr == w && t.nv >= per_lane && (!best || t.nv < best->nv)) {
        best = &t;
      }
    }
  }
  if (best) return best;
  for (int i = 0; i < table->count; ++i) {  // any covering tile
    const Tile& t = table->tiles[i];
    if (t.vec == vec && (int64_t)64 * t.wpr * t.nv >= nvec) return &t;
  }
  return nullptr;
}

// Grid limit per launch; larger row counts are split into several launches.
constexpr int64_t kMaxBlocksPerLaunch = int64_t(1) << 22;

// The launch plan of one norm call: the access width and the tile.  The
// arguments are checked first; `cus` <= 0 then reads the current device's
// CU count (the first HIP call), otherwise no HIP call is made.
struct Plan {
  int vec = 0;
  const Tile* tile = nullptr;
};

int plan_norm(const Request& r, int cus, Plan* out) {
  const bool fp8 = (r.kind & 6) != 0;

  // ---- argument checks (no HIP call before they pass) ----
  if (r.dtype != ARN_BF16 && r.dtype != ARN_FP16) return ARN_EINVAL;
  if (r.rows < 0 || r.hidden <= 0) return ARN_EINVAL;
  if (r.x_stride < r.hidden || r.out_stride < r.hidden) return ARN_EINVAL;
  if ((r.kind & 1) && r.res_stride < r.hidden) return ARN_EINVAL;
  if (!(r.eps >= 0.0f) || !std::isfinite(r.eps)) return ARN_EINVAL;
  if (r.var_cols < 0 || r.var_cols > r.hidden) return ARN_EINVAL;
  if (r.parts && (r.nparts < 1 || r.nparts > arn::kMaxParts)) return ARN_EINVAL;
  if (r.rows == 0) return ARN_OK;
  if (!r.out || !r.x) return ARN_EINVAL;
  for (int g = 0; g < r.nparts; ++g) {
    if (!r.parts[g] || !aligned(r.parts[g], 2)) return ARN_EINVAL;
    if (g > 0 && r.parts[g] == r.out) return ARN_EINVAL;
    if (r.res && r.parts[g] == r.res) return ARN_EINVAL;
  }
  if ((r.kind & 1) && !r.res) return ARN_EINVAL;
  if (fp8 && (!r.scale || !aligned(r.scale, 4))) return ARN_EINVAL;
  if (!aligned(r.x, 2) || (r.res && !aligned(r.res, 2)) || (r.w && !aligned(r.w, 2)) ||
      (!fp8 && !aligned(r.out, 2))) {
    return ARN_EINVAL;
  }
  // Aliasing: out may be x itself (same stride, 16-bit output); the
  // residual may alias neither.
  if (r.res && (r.res == r.x || r.res == r.out)) return ARN_EINVAL;
  if (r.out == r.x && (fp8 || r.out_stride != r.x_stride)) return ARN_EINVAL;
  if (r.hidden > (int64_t)1 << 30) return ARN_EUNSUPPORTED;

  const int vec = choose_vec(r);
  const int64_t nvec = r.hidden / vec;
  const TileTable* table = r.parts ? sum_table_for(r.kind, r.dtype) : table_for(r.kind, r.dtype);
  // Compact tiles (choose_tile): plain kinds up to four vectors per lane;
  // the fused dynamic-e4m3 kind and the all-reduce form over two or three
  // parts up to two.
  int compact = 0;
  if (r.parts) {
    if (r.nparts < 4) compact = 2;
  } else if (!(r.kind & arn::kFused)) {
    compact = 4;
  } else if (r.kind == arn::kFusedFp8Dynamic) {
    compact = 2;
  }
  if (cus <= 0) cus = cu_count();
  int waves = 0;
  if ((r.kind & arn::kFused) && !r.parts && vec == 8 && nvec > 512 && nvec <= 1024 &&
      r.rows <= 2 * (int64_t)cus) {
    if (2 * r.rows > cus) {
      waves = (4 * r.rows > 5 * (int64_t)cus && nvec > 768) ? 2 : 4;
    } else if (r.dtype == ARN_FP16) {
      waves = 4;
    }
  }
  const Tile* tile = choose_tile(table, vec, nvec, r.rows, cus, r.nparts >= 4, compact, waves);
  if (!tile) return ARN_EUNSUPPORTED;
  out->vec = vec;
  out->tile = tile;
  return ARN_OK;
}

// The blocks of the last launch of a call (calls past the grid limit are
// split into several launches).
int64_t last_grid(int64_t rows, const Tile* tile) {
  const int64_t rows_per_launch = kMaxBlocksPerLaunch * tile->rpb;
  const int64_t n = rows - (rows - 1) / rows_per_launch * rows_per_launch;
  return (n + tile->rpb - 1) / tile->rpb;
}

int describe_plan(const Request& r, const Plan& p, int64_t grid, char* buf, size_t len) {
  return std::snprintf(buf, len, "%s%s/%s/vec%d/wpr%d/nv%d/rpb%d/grid%lld",
                       r.parts ? "sum_" : "", kKindNames[r.kind],
                       r.dtype == ARN_BF16 ? "bf16" : "fp16", p.vec, p.tile->wpr, p.tile->nv,
                       p.tile->rpb, (long long)grid);
}

// The request of an arn_norm descriptor (its struct size and output format
// checked here, the rest by plan_norm).
int norm_request(const arn_norm_args* p, Request* r) {
  if (!p || p->struct_size < sizeof(arn_norm_args)) return ARN_EINVAL;
  int kind;
  switch (p->out_format) {
    case ARN_OUT_16BIT:
      kind = arn::kPlain;
      break;
    case ARN_OUT_FP8_STATIC:
      kind = arn::kPlainFp8Static;
      break;
    case ARN_OUT_FP8_DYNAMIC:
      kind = arn::kPlainFp8Dynamic;
      break;
    default:
      return ARN_EINVAL;
  }
  if (p->residual) kind |= arn::kFused;
  *r = Request{kind,        p->dtype,           p->out,    p->out_stride,
               p->x,        p->x_stride,        p->residual, p->residual_stride,
               p->weight,   kind & 6 ? p->scale : nullptr, p->eps, p->rows,
               p->hidden,   p->stream,          p->variance_size};
  return ARN_OK;
}

int run(const Request& r) {
  const bool fp8 = (r.kind & 6) != 0;
  const bool dynamic = (r.kind & 4) != 0;
  Plan p;
  const int st = plan_norm(r, 0, &p);
  if (st != ARN_OK || r.rows == 0) return st;
  const Tile* tile = p.tile;

  const int esize_out = fp8 ? 1 : 2;
  const int64_t rows_per_launch = kMaxBlocksPerLaunch * tile->rpb;
  int64_t done = 0;
  int64_t grid = 0;
  while (done < r.rows) {
    const int64_t n = (r.rows - done < rows_per_launch) ? r.rows - done : rows_per_launch;
    Args a;
    a.out = static_cast<char*>(r.out) + done * r.out_stride * esize_out;
    a.out_stride = r.out_stride;
    a.x = static_cast<const char*>(r.x) + done * r.x_stride * 2;
    a.x_stride = r.x_stride;
    a.res = r.res ? static_cast<char*>(r.res) + done * r.res_stride * 2 : nullptr;
    a.res_stride = r.res_stride;
    a.w = r.w;
    a.scale = dynamic ? r.scale + done : r.scale;
    a.rows = n;
    a.hidden = (int32_t)r.hidden;
    a.eps = r.eps;
    a.var_cols = (int32_t)(r.var_cols > 0 ? r.var_cols : r.hidden);
    a.inv_var = 1.0f / (float)a.var_cols;
    a.nparts = r.nparts;
    for (int g = 0; g < arn::kMaxParts; ++g) {
      a.parts[g] = g < r.nparts ? static_cast<const char*>(r.parts[g]) + done * r.x_stride * 2
                                : nullptr;
    }

    grid = (n + tile->rpb - 1) / tile->rpb;
    void* params[] = {&a};
    const hipError_t e = hipLaunchKernel(tile->fn, dim3((unsigned)grid),
                                         dim3(64u * tile->wpr * tile->rpb), params, 0, r.stream);
    if (e != hipSuccess) return ARN_ELAUNCH;
    done += n;
  }

  g_last_plan_len = describe_plan(r, p, grid, g_last_plan, sizeof(g_last_plan));
  return ARN_OK;
}

// SwiGLU: out = silu(gate) * up over d columns per row.
int run_glu(int mode, int dtype, void* out, int64_t out_stride, float* scale, const void* gate,
            int64_t gate_stride, const void* up, int64_t up_stride, int64_t rows, int64_t d,
            hipStream_t stream) {
  const bool fp8 = mode != arn::kGluPlain;
  if (dtype != ARN_BF16 && dtype != ARN_FP16) return ARN_EINVAL;
  if (rows < 0 || d <= 0) return ARN_EINVAL;
  if (gate_stride < d || up_stride < d || out_stride < d) return ARN_EINVAL;
  if (rows == 0) return ARN_OK;
  if (!out || !gate || !up) return ARN_EINVAL;
  if (fp8 && (!scale || !aligned(scale, 4))) return ARN_EINVAL;
  if (!aligned(gate, 2) || !aligned(up, 2) || (!fp8 && !aligned(out, 2))) return ARN_EINVAL;
  if (out == gate || out == up) return ARN_EINVAL;
  if (d > (int64_t)1 << 30) return ARN_EUNSUPPORTED;

  int vec = 1;
  for (int v = 8; v > 1; v /= 2) {
    const uintptr_t b16 = 2u * v;
    bool ok = d % v == 0 && gate_stride % v == 0 && up_stride % v == 0 && out_stride % v == 0 &&
              aligned(gate, b16) && aligned(up, b16) && aligned(out, fp8 ? v : b16);
    if (ok) {
      vec = v;
      break;
    }
  }
  const int64_t nvec = d / vec;
  // Compact tiles up to two vectors per lane (choose_tile).
  const Tile* tile = choose_tile(glu_table_for(mode, dtype), vec, nvec, rows, cu_count(), false, 2);
  if (!tile) return ARN_EUNSUPPORTED;

  const int esize_out = fp8 ? 1 : 2;
  const int64_t rows_per_launch = kMaxBlocksPerLaunch * tile->rpb;
  int64_t done = 0;
  int64_t grid = 0;
  while (done < rows) {
    const int64_t n = (rows - done < rows_per_launch) ? rows - done : rows_per_launch;
    arn::GluArgs a;
    a.out = static_cast<char*>(out) + done * out_stride * esize_out;
    a.out_stride = out_stride;
    a.gate = static_cast<const char*>(gate) + done * gate_stride * 2;
    a.gate_stride = gate_stride;
    a.up = static_cast<const char*>(up) + done * up_stride * 2;
    a.up_stride = up_stride;
    a.scale = mode == arn::kGluDynamic ? scale + done : scale;
    a.rows = n;
    a.d = (int32_t)d;
    grid = (n + tile->rpb - 1) / tile->rpb;
    void* params[] = {&a};
    const hipError_t e = hipLaunchKernel(tile->fn, dim3((unsigned)grid),
                                         dim3(64u * tile->wpr * tile->rpb), params, 0, stream);
    if (e != hipSuccess) return ARN_ELAUNCH;
    done += n;
  }
  g_last_plan_len = std::snprintf(g_last_plan, sizeof(g_last_plan),
                                  "%s/%s/vec%d/wpr%d/nv%d/rpb%d/grid%lld", kGluNames[mode],
                                  dtype == ARN_BF16 ? "bf16" : "fp16", vec, tile->wpr, tile->nv,
                                  tile->rpb, (long long)grid);
  return ARN_OK;
}

// Forced GEMM shape (arn_set_gemm_config); 0 = automatic.  nt << 8 | waves.
thread_local int g_forced_gemm = 0;

// GEMM shape, from sweeps of decode projections on MI355X (N 2304..16384,
// K 2048..16384, M 1..64).  The weight stream wants about one block per CU
// or more: the widest column tile that still gives at least 3/4 of a block
// per CU.  Wide tiles matter more as M grows: every block reads all of A
// (M x K), so A's share of the load traffic per block is M / (16 NT) of the
// weight's.  With one row tile, K is split over eight waves once each keeps
// four or more 128-wide k steps, else over four (16 waves measured 1-12%
// slower at K = 8192-16384, most with one column tile: the QKV shard
// 2304 x 16384 at M = 1 takes 9.1 us with 8 waves, 10.3 with 16); with two
// or four row tiles the accumulators and operands of a wave fill its
// registers, and four waves per block do best.
const GemmCfg* find_gemm(const GemmTable* table, int mt, int nt, int waves);

const GemmCfg* choose_gemm(const GemmTable* table, bool pre, int mt, int64_t n, int64_t k,
                           int cus) {
  const int forced = g_forced_gemm;
  auto find = [&](int nt, int waves) { return find_gemm(table, mt, nt, waves); };
  if (forced != 0) return find(forced >> 8, forced & 0xFF);
  const int64_t ksteps = (k + 127) / 128;
  const int64_t want_blocks = (3 * (int64_t)cus) / 4;
  auto blocks = [&](int nt) { return (n + 16 * nt - 1) / (16 * nt); };
  int nt = 1;
  if (blocks(4) >= want_blocks) {
    nt = 4;
  } else if (blocks(2) >= want_blocks) {
    nt = 2;
  }
  // A grid just past one block per CU leaves a few CUs a second block while
  // the rest wait: take the next wider tile instead (one block on every
  // other CU or so).  N = 4608 at K = 16384, M = 1: 288 blocks 18.9 us,
  // 144 blocks 15.4; N = 9216: 31.1 and 27.1.
  if (nt < 4 && blocks(nt) > cus && blocks(nt) * 4 <= (int64_t)cus * 5) nt *= 2;
  int waves = 4;
  if (mt == 1 && ksteps >= 32) waves = 8;
  // A row-major weight goes through LDS on its way to the operands: with
  // several column tiles and a long K, more waves hide that (gate_up at
  // M = 1: 38.2 us with 16 waves, 40.4 with 8).
  if (mt == 1 && !pre && nt >= 2 && ksteps >= 64) waves = 16;
  return find(nt, waves);
}

// Largest weight slice one GEMM launch addresses (buffer records are 32-bit).
constexpr int64_t kMaxGemmBBytes = int64_t(1) << 31;
// Largest K of a pre-shuffled weight: a panel of at least 4 column tiles
// (ceil(K/128) 2 KiB tiles each) stays within 1 GiB.
constexpr int64_t kMaxPreshuffleK = int64_t(1) << 23;

int64_t preshuffled_bytes(int64_t n, int64_t k) {
  return ((n + 15) / 16) * ((k + 127) / 128) * 2048;
}

// Split-K workspace layout, a function of the workspace size alone so that
// calls of different shapes sharing one workspace agree on where the
// counters live: the partial tiles from the start, the int32 counters (one
// per column tile, zero between calls) in the last ~1/512 of it.  The size
// for m x n outputs covers up to kMaxSplits splits of every compiled shape.
constexpr int kMaxSplits = 8;
int64_t round_up(int64_t v, int64_t a) { return (v + a - 1) / a * a; }
int64_t partial_bound(int64_t m, int64_t n) {
  const int64_t mpad = m <= 16 ? 16 : (m <= 32 ? 32 : 64);
  return (int64_t)kMaxSplits * mpad * round_up(n, 64) * 4;
}
int64_t workspace_bytes(int64_t m, int64_t n) {
  const int64_t p = partial_bound(m, n);
  return round_up(p + round_up(p / 256, 256) + 512, 256);
}
// Counter region of a workspace of `bytes` (both 256-byte multiples):
// [usable - counters, usable).
int64_t ws_usable(size_t bytes) { return (int64_t)bytes / 256 * 256; }
int64_t ws_counter_bytes(size_t bytes) { return round_up(ws_usable(bytes) / 512 + 1, 256); }

// Forced number of K splits (arn_set_gemm_splits); 0 = automatic.
thread_local int g_forced_splits = 0;

const GemmCfg* find_gemm(const GemmTable* table, int mt, int nt, int waves) {
  for (int i = 0; i < table->count; ++i) {
    const GemmCfg& g = table->cfgs[i];
    if (g.mt == mt && g.nt == nt && g.waves == waves) return &g;
  }
  return nullptr;
}

// With a workspace: when N is too small for one column tile per CU (the
// shape choice fell back to 16-column tiles, e.g. a QKV projection shard)
// and M >= 8, use 32-column tiles of 8 waves and split K so that the grid
// holds about one block per CU.  From sweeps on MI355X: 2304 x 16384 at
// M = 16 / 32 / 64 runs 14-38% faster this way; at M = 1 the split costs
// more than it gains, and shapes with enough columns gain nothing from a
// split and keep their shape.
const GemmCfg* choose_split(const GemmTable* table, const GemmCfg* cfg, int64_t m, int64_t n,
                            int cus, int* splits) {
  const int forced = g_forced_splits;
  if (forced > 0) {
    *splits = forced;
    return cfg;
  }
  *splits = 1;
  if (g_forced_gemm != 0 || cfg->nt != 1 || m < 8) return cfg;
  const GemmCfg* wide = find_gemm(table, cfg->mt, 2, 8);
  const int64_t blocks = (n + 31) / 32;
  const int64_t sp = blocks > 0 ? cus / blocks : 1;
  if (!wide || sp < 2) return cfg;
  *splits = (int)(sp < kMaxSplits ? sp : kMaxSplits);
  return wide;
}

// pre: b is the pre-shuffled copy (ldb ignored), else N x K row-major.
// workspace (may be null: no split) holds workspace_bytes(m, n) bytes whose
// counters are zero.
int run_gemm(bool pre, void* c, int64_t ldc, int out_dtype, const uint8_t* a, int64_t lda,
             const float* scale_a, int a_per_row, const uint8_t* b, int64_t ldb,
             const float* scale_b, int b_per_row, int64_t m, int64_t n, int64_t k,
             void* workspace, size_t ws_bytes, hipStream_t stream) {
  if (out_dtype != ARN_BF16 && out_dtype != ARN_FP16) return ARN_EINVAL;
  if (m < 0 || n < 0 || k <= 0) return ARN_EINVAL;
  if (lda < k || (!pre && ldb < k) || ldc < n) return ARN_EINVAL;
  if (m == 0 || n == 0) return ARN_OK;
  if (!c || !a || !b || !scale_a || !scale_b) return ARN_EINVAL;
  if (!aligned(c, 2) || !aligned(scale_a, 4) || !aligned(scale_b, 4)) return ARN_EINVAL;
  if (workspace && (!aligned(workspace, 256) || (int64_t)ws_bytes < workspace_bytes(m, n))) {
    return ARN_EINVAL;
  }
  // Served shapes: up to 64 activation rows, K a multiple of 16, 16-byte
  // aligned operand rows.
  if (m > 64 || k % 16 != 0 || lda % 16 != 0 || !aligned(a, 16) || !aligned(b, 16) ||
      m * lda > kMaxGemmBBytes) {
    return ARN_EUNSUPPORTED;
  }
  // (A block addresses up to 64 weight rows through one buffer record.)
  if (pre ? k > kMaxPreshuffleK : (ldb % 16 != 0 || ldb > kMaxGemmBBytes / 64)) {
    return ARN_EUNSUPPORTED;
  }
  const int mt = m <= 16 ? 1 : (m <= 32 ? 2 : 4);
  const GemmTable* table = &ARN_GEMM_TABLE_NAME(0);
  if (out_dtype == ARN_FP16) table = &ARN_GEMM_TABLE_NAME(1);
  const int cus = cu_count();
  const GemmCfg* cfg = choose_gemm(table, pre, mt, n, k, cus);
  if (!cfg) return ARN_EUNSUPPORTED;
  const int64_t nsteps = (k + 127) / 128;

  int splits = 1;
  if (workspace) {
    cfg = choose_split(table, cfg, m, n, cus, &splits);
    if (splits > kMaxSplits) splits = kMaxSplits;
    if (splits > nsteps) splits = (int)nsteps;
    if (splits < 1) splits = 1;
  }
  const int nt = cfg->nt;
  const int64_t tile_cols = 16 * nt;
  const int64_t k_tile = (int64_t)cfg->mt * nt * 256;  // outputs per block
  const int steps_per_split = (int)((nsteps + splits - 1) / splits);
  splits = (int)((nsteps + steps_per_split - 1) / steps_per_split);  // no empty split
  if (splits > 1) {
    // Guaranteed by the size check above; kept as a guard on the layout.
    const int64_t tiles = (n + tile_cols - 1) / tile_cols;
    if (tiles * splits * k_tile * 4 > ws_usable(ws_bytes) - ws_counter_bytes(ws_bytes) ||
        tiles * 4 > ws_counter_bytes(ws_bytes)) {
      return ARN_EINVAL;
    }
  }
  float* partial = static_cast<float*>(workspace);
  int32_t* counters =
      workspace ? reinterpret_cast<int32_t*>(static_cast<char*>(workspace) +
                                             ws_usable(ws_bytes) - ws_counter_bytes(ws_bytes))
                : nullptr;

  // Split N so that each launch's weight slice stays under 2 GiB (row-major)
  // or covers one panel of the pre-shuffled copy.
  int64_t rows_per_launch = pre ? panel_tiles_for(nsteps) * 16 : (kMaxGemmBBytes / ldb);
  rows_per_launch = rows_per_launch / tile_cols * tile_cols;
  if (rows_per_launch <= 0) return ARN_EUNSUPPORTED;
  int64_t done = 0;
  int64_t grid = 0;
  while (done < n) {
    const int64_t cols = (n - done < rows_per_launch) ? n - done : rows_per_launch;
    const int64_t tile0 = done / tile_cols;
    GemmArgs g;
    g.c = static_cast<char*>(c) + done * 2;
    g.ldc = ldc;
    g.a = a;
    g.lda = lda;
    g.scale_a = scale_a;
    g.b = pre ? b + (done / 16) * nsteps * 2048 : b + done * ldb;  // a panel starts there
    g.ldb = pre ? 0 : ldb;
    g.scale_b = b_per_row ? scale_b + done : scale_b;
    g.m = m;
    g.n = cols;
    g.k = k;
    g.a_per_row = a_per_row ? 1 : 0;
    g.b_per_row = b_per_row ? 1 : 0;
    g.splits = splits;
    g.steps_per_split = steps_per_split;
    g.partial = splits > 1 ? partial + tile0 * splits * k_tile : nullptr;
    g.counters = splits > 1 ? counters + tile0 : nullptr;
    grid = (cols + tile_cols - 1) / tile_cols;
    void* params[] = {&g};
    const hipError_t e = hipLaunchKernel(pre ? cfg->fn_pre : cfg->fn,
                                         dim3((unsigned)grid, (unsigned)splits),
                                         dim3(64u * cfg->waves), params, 0, stream);
    if (e != hipSuccess) return ARN_ELAUNCH;
    done += cols;
  }
  g_last_plan_len = std::snprintf(g_last_plan, sizeof(g_last_plan),
                                  "fp8_gemm%s/%s/mt%d/nt%d/waves%d/splits%d/grid%lld",
                                  pre ? "_preshuffled" : "",
                                  out_dtype == ARN_BF16 ? "bf16" : "fp16", cfg->mt, cfg->nt,
                                  cfg->waves, splits, (long long)grid);
  return ARN_OK;
}

int run_preshuffle(uint8_t* dst, const uint8_t* b, int64_t ldb, int64_t n, int64_t k,
                   hipStream_t stream) {
  if (n < 0 || k <= 0 || ldb < k) return ARN_EINVAL;
  if (n == 0) return ARN_OK;
  if (!dst || !b) return ARN_EINVAL;
  if (!aligned(dst, 16) || k > kMaxPreshuffleK) return ARN_EUNSUPPORTED;
  const int64_t pieces = preshuffled_bytes(n, k) / 16;
  const int64_t grid = (pieces + 255) / 256;
  if (grid > int64_t(0x7FFFFFFF)) return ARN_EUNSUPPORTED;
  arn::PreshuffleArgs p;
  p.dst = dst;
  p.src = b;
  p.ldb = ldb;
  p.n = n;
  p.k = k;
  p.ntiles = (n + 15) / 16;
  p.nsteps = (k + 127) / 128;
  p.panel_tiles = panel_tiles_for(p.nsteps);
  p.aligned = (ldb % 16 == 0 && aligned(b, 16)) ? 1 : 0;
  void* params[] = {&p};
  const hipError_t e =
      hipLaunchKernel(arn_preshuffle_fn, dim3((unsigned)grid), dim3(256u), params, 0, stream);
  return e == hipSuccess ? ARN_OK : ARN_ELAUNCH;
}

// ---------------------------------------------------------------------------
// Device scratch of arn_fp8_gemm_preshuffled_noalloc: the split-K partial
// tiles and tile counters, in a file-scope array instead of a caller's
// workspace, for callers that cannot allocate.  Every GPU the library runs
// on holds its own copy until the process ends; its address is taken once
// per device with hipGetSymbolAddress (the array's name is only a host-side
// stand-in), and that address is what the kernels receive.
// ---------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[ARN_NOALLOC_SCRATCH_BYTES];

__global__ void zero_words(uint32_t* p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

struct ScratchSlot {
  std::once_flag once;
  void* ptr = nullptr;
  int status = ARN_ELAUNCH;
};
ScratchSlot g_scratch[64];

// The current device's scratch address.  On the first call for a device the
// address is looked up and the counter region is cleared by a small kernel
// on `stream` (no memset node, so a capturing caller records a kernel);
// every completed call leaves the counters at zero again.
int scratch_for_current_device(hipStream_t stream, void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return ARN_ELAUNCH;
  ScratchSlot& slot = g_scratch[dev];
  std::call_once(slot.once, [&] {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return;
    const size_t bytes = ARN_NOALLOC_SCRATCH_BYTES;
    const int64_t cbytes = ws_counter_bytes(bytes);
    uint32_t* counters =
        reinterpret_cast<uint32_t*>(static_cast<char*>(ptr) + ws_usable(bytes) - cbytes);
    const int64_t words = cbytes / 4;
    void* params[] = {&counters, const_cast<int64_t*>(&words)};
    if (hipLaunchKernel((const void*)&zero_words, dim3((unsigned)((words + 255) / 256)),
                        dim3(256u), params, 0, stream) != hipSuccess) {
      return;
    }
    slot.ptr = ptr;
    slot.status = ARN_OK;
  });
  *out = slot.ptr;
  return slot.status;
}

}  // namespace

extern "C" {

int arn_fp8_gemm_preshuffled_noalloc(void* c, int64_t ldc, int out_dtype, const uint8_t* a,
                                     int64_t lda, const float* scale_a, int a_per_row,
                                     const uint8_t* b_shuffled, const float* scale_b,
                                     int b_per_row, int64_t m, int64_t n, int64_t k,
                                     hipStream_t stream) {
  // The argument checks of the workspace entry point, then the size limit,
  // all before any HIP call.
  if (out_dtype != ARN_BF16 && out_dtype != ARN_FP16) return ARN_EINVAL;
  if (m < 0 || n < 0 || k <= 0 || lda < k || ldc < n) return ARN_EINVAL;
  if (m == 0 || n == 0) return ARN_OK;
  if (!c || !a || !b_shuffled || !scale_a || !scale_b) return ARN_EINVAL;
  if (workspace_bytes(m, n) > (int64_t)ARN_NOALLOC_SCRATCH_BYTES) return ARN_EUNSUPPORTED;
  void* ws = nullptr;
  const int st = scratch_for_current_device(stream, &ws);
  if (st != ARN_OK) return st;
  return run_gemm(true, c, ldc, out_dtype, a, lda, scale_a, a_per_row, b_shuffled, 0, scale_b,
                  b_per_row, m, n, k, ws, ARN_NOALLOC_SCRATCH_BYTES, stream);
}

int arn_fp8_gemm(void* c, int64_t ldc, int out_dtype, const uint8_t* a, int64_t lda,
                 const float* scale_a, int a_per_row, const uint8_t* b, int64_t ldb,
                 const float* scale_b, int b_per_row, int64_t m, int64_t n, int64_t k,
                 hipStream_t stream) {
  return run_gemm(false, c, ldc, out_dtype, a, lda, scale_a, a_per_row, b, ldb, scale_b,
                  b_per_row, m, n, k, nullptr, 0, stream);
}

int arn_fp8_gemm_ws(void* c, int64_t ldc, int out_dtype, const uint8_t* a, int64_t lda,
                    const float* scale_a, int a_per_row, const uint8_t* b, int64_t ldb,
                    const float* scale_b, int b_per_row, int64_t m, int64_t n, int64_t k,
                    void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return run_gemm(false, c, ldc, out_dtype, a, lda, scale_a, a_per_row, b, ldb, scale_b,
                  b_per_row, m, n, k, workspace, workspace_bytes, stream);
}

int64_t arn_fp8_gemm_workspace_bytes(int64_t m, int64_t n, int64_t k) {
  if (m < 0 || n < 0 || k <= 0) return -1;
  return workspace_bytes(m, n);
}

int64_t arn_fp8_weight_preshuffled_bytes(int64_t n, int64_t k) {
  if (n < 0 || k <= 0) return -1;
  return preshuffled_bytes(n, k);
}

int arn_fp8_weight_preshuffle(uint8_t* dst, const uint8_t* b, int64_t ldb, int64_t n, int64_t k,
                              hipStream_t stream) {
  return run_preshuffle(dst, b, ldb, n, k, stream);
}

int arn_fp8_gemm_preshuffled(void* c, int64_t ldc, int out_dtype, const uint8_t* a, int64_t lda,
                             const float* scale_a, int a_per_row, const uint8_t* b_shuffled,
                             const float* scale_b, int b_per_row, int64_t m, int64_t n, int64_t k,
                             hipStream_t stream) {
  return run_gemm(true, c, ldc, out_dtype, a, lda, scale_a, a_per_row, b_shuffled, 0, scale_b,
                  b_per_row, m, n, k, nullptr, 0, stream);
}

int arn_fp8_gemm_preshuffled_ws(void* c, int64_t ldc, int out_dtype, const uint8_t* a,
                                int64_t lda, const float* scale_a, int a_per_row,
                                const uint8_t* b_shuffled, const float* scale_b, int b_per_row,
                                int64_t m, int64_t n, int64_t k, void* workspace,
                                size_t workspace_bytes, hipStream_t stream) {
  return run_gemm(true, c, ldc, out_dtype, a, lda, scale_a, a_per_row, b_shuffled, 0, scale_b,
                  b_per_row, m, n, k, workspace, workspace_bytes, stream);
}


int arn_silu_and_mul(void* out, int64_t out_stride, const void* gate, int64_t gate_stride,
                     const void* up, int64_t up_stride, int64_t rows, int64_t d, int dtype,
                     hipStream_t stream) {
  return run_glu(arn::kGluPlain, dtype, out, out_stride, nullptr, gate, gate_stride, up,
                 up_stride, rows, d, stream);
}

int arn_silu_and_mul_fp8(uint8_t* out, int64_t out_stride, float* scale, int fp8_mode,
                         const void* gate, int64_t gate_stride, const void* up, int64_t up_stride,
                         int64_t rows, int64_t d, int dtype, hipStream_t stream) {
  if (fp8_mode != ARN_FP8_STATIC && fp8_mode != ARN_FP8_DYNAMIC) return ARN_EINVAL;
  return run_glu(fp8_mode == ARN_FP8_STATIC ? arn::kGluStatic : arn::kGluDynamic, dtype, out,
                 out_stride, scale, gate, gate_stride, up, up_stride, rows, d, stream);
}


int arn_rmsnorm(void* out, int64_t out_stride, const void* x, int64_t x_stride,
                const void* weight, float eps, int64_t rows, int64_t hidden, int dtype,
                hipStream_t stream) {
  Request r{arn::kPlain, dtype, out,     out_stride, x,    x_stride, nullptr,
            0,           weight, nullptr, eps,       rows, hidden,   stream};
  return run(r);
}

int arn_fused_add_rmsnorm(void* out, int64_t out_stride, const void* x, int64_t x_stride,
                          void* residual, int64_t residual_stride, const void* weight, float eps,
                          int64_t rows, int64_t hidden, int dtype, hipStream_t stream) {
  Request r{arn::kFused, dtype,  out,     out_stride, x,    x_stride, residual,
            residual_stride, weight, nullptr, eps,     rows, hidden,   stream};
  return run(r);
}

int arn_rmsnorm_fp8(uint8_t* out, int64_t out_stride, float* scale, int fp8_mode, const void* x,
                    int64_t x_stride, const void* weight, float eps, int64_t rows, int64_t hidden,
                    int dtype, hipStream_t stream) {
  if (fp8_mode != ARN_FP8_STATIC && fp8_mode != ARN_FP8_DYNAMIC) return ARN_EINVAL;
  const int kind = fp8_mode == ARN_FP8_STATIC ? arn::kPlainFp8Static : arn::kPlainFp8Dynamic;
  Request r{kind, dtype,  out,   out_stride, x,    x_stride, nullptr,
            0,    weight, scale, eps,        rows, hidden,   stream};
  return run(r);
}

int arn_fused_add_rmsnorm_fp8(uint8_t* out, int64_t out_stride, float* scale, int fp8_mode,
                              const void* x, int64_t x_stride, void* residual,
                              int64_t residual_stride, const void* weight, float eps,
                              int64_t rows, int64_t hidden, int dtype, hipStream_t stream) {
  if (fp8_mode != ARN_FP8_STATIC && fp8_mode != ARN_FP8_DYNAMIC) return ARN_EINVAL;
  const int kind = fp8_mode == ARN_FP8_STATIC ? arn::kFusedFp8Static : arn::kFusedFp8Dynamic;
  Request r{kind,           dtype,  out,   out_stride, x,    x_stride, residual,
            residual_stride, weight, scale, eps,        rows, hidden,   stream};
  return run(r);
}

int arn_norm(const arn_norm_args* p) {
  Request r{};
  const int st = norm_request(p, &r);
  return st != ARN_OK ? st : run(r);
}

int arn_norm_plan(const arn_norm_args* p, int compute_units, char* buf, size_t len) {
  if (buf && len > 0) buf[0] = '\0';
  if (compute_units <= 0) return ARN_EINVAL;
  Request r{};
  int st = norm_request(p, &r);
  if (st != ARN_OK) return st;
  Plan pl;
  st = plan_norm(r, compute_units, &pl);
  if (st != ARN_OK || r.rows == 0) return st;
  if (buf && len > 0) describe_plan(r, pl, last_grid(r.rows, pl.tile), buf, len);
  return ARN_OK;
}

int arn_sum_add_rmsnorm(const arn_sum_norm_args* p) {
  if (!p || p->struct_size < sizeof(arn_sum_norm_args)) return ARN_EINVAL;
  if (!p->parts) return ARN_EINVAL;
  int kind;
  switch (p->out_format) {
    case ARN_OUT_16BIT:
      kind = arn::kPlain;
      break;
    case ARN_OUT_FP8_STATIC:
      kind = arn::kPlainFp8Static;
      break;
    case ARN_OUT_FP8_DYNAMIC:
      kind = arn::kPlainFp8Dynamic;
      break;
    default:
      return ARN_EINVAL;
  }
  if (p->residual) kind |= arn::kFused;
  Request r{kind,      p->dtype,  p->out,    p->out_stride, p->nparts > 0 ? p->parts[0] : nullptr,
            p->parts_stride, p->residual, p->residual_stride, p->weight,
            kind & 6 ? p->scale : nullptr, p->eps, p->rows, p->hidden, p->stream, 0,
            p->parts, p->nparts};
  return run(r);
}

const char* arn_status_str(int status) {
  switch (status) {
    case ARN_OK:
      return "ok";
    case ARN_EINVAL:
      return "invalid argument";
    case ARN_EUNSUPPORTED:
      return "unsupported shape or layout";
    case ARN_ELAUNCH:
      return "kernel launch failed";
    default:
      return "unknown status";
  }
}

int arn_abi_version(void) { return ARN_ABI_VERSION; }

int arn_set_tile(int waves_per_row, int vec_per_lane) {
  if (waves_per_row == 0 && vec_per_lane == 0) {
    g_forced_tile = 0;
    return ARN_OK;
  }
  // The tile must exist in the tables (all tables list the same shapes).
  const TileTable* t = table_for(arn::kPlain, ARN_BF16);
  for (int i = 0; i < t->count; ++i) {
    if (t->tiles[i].wpr == waves_per_row && t->tiles[i].nv == vec_per_lane) {
      g_forced_tile = (waves_per_row << 8) | vec_per_lane;
      return ARN_OK;
    }
  }
  return ARN_EINVAL;
}

int arn_set_gemm_config(int col_tiles, int waves) {
  if (col_tiles == 0 && waves == 0) {
    g_forced_gemm = 0;
    return ARN_OK;
  }
  const GemmTable* t = &ARN_GEMM_TABLE_NAME(0);
  for (int i = 0; i < t->count; ++i) {
    if (t->cfgs[i].nt == col_tiles && t->cfgs[i].waves == waves) {
      g_forced_gemm = (col_tiles << 8) | waves;
      return ARN_OK;
    }
  }
  return ARN_EINVAL;
}

int arn_set_gemm_splits(int splits) {
  if (splits < 0 || splits > kMaxSplits) return ARN_EINVAL;
  g_forced_splits = splits;
  return ARN_OK;
}

int arn_last_plan(char* buf, size_t len) {
  if (buf && len > 0) {
    std::strncpy(buf, g_last_plan, len - 1);
    buf[len - 1] = '\0';
  }
  return g_last_plan_len;
}

}  // extern "C"
