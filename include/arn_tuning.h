/*
 * arn_tuning.h -- test and tuning aids of the library declared in arn.h.
 *
 * Not needed for normal use.  The tests and the benchmark use them to force
 * one compiled kernel shape at a time and to read back which shape a call
 * took.  Every setting here is held PER CALLING THREAD: it changes only the
 * later calls that same thread makes, and no other thread ever sees it, so
 * a forgotten reset cannot change or refuse another thread's calls.  A new
 * thread starts with automatic selection everywhere.
 */
#ifndef ARN_TUNING_H
#define ARN_TUNING_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * arn_set_tile forces the kernel shape of the calling thread's later norm,
 * all-reduce-form and SwiGLU calls: waves_per_row (1, 2, 4, 8, 16) 64-lane
 * waves share one row, and each lane keeps up to vec_per_lane vectors of the
 * row in registers.  A call whose shape the forced tile cannot serve returns
 * ARN_EUNSUPPORTED.  (0, 0) restores automatic selection.  Returns
 * ARN_EINVAL for a tile that is not compiled (the setting is then left as
 * it was).
 */
int arn_set_tile(int waves_per_row, int vec_per_lane);

/*
 * arn_set_gemm_config forces the shape of the calling thread's later GEMM
 * calls: each block computes col_tiles x 16 output columns (1, 2 or 4) with
 * K split over `waves` waves (4, 8 or 16).  A call whose row tiling has no
 * such compiled shape returns ARN_EUNSUPPORTED.  (0, 0) restores automatic
 * selection; a shape never compiled returns ARN_EINVAL.
 */
int arn_set_gemm_config(int col_tiles, int waves);

/*
 * arn_set_gemm_splits forces the number of K splits (1..8) of the calling
 * thread's later workspace GEMM calls (capped by the number of 128-wide k
 * steps); 0 restores automatic selection.  ARN_EINVAL outside 0..8.
 */
int arn_set_gemm_splits(int splits);

/*
 * arn_last_plan copies into buf (size len, always NUL-terminated when
 * len > 0) a description of the kernel the calling thread's last successful
 * launch used, e.g. "fused_add/bf16/vec8/wpr8/nv2/rpb1/grid4096".  Returns
 * the full length of the description (0 before the thread's first launch).
 */
int arn_last_plan(char *buf, size_t len);

/*
 * arn_norm_plan answers, without any HIP call and without launching, which
 * kernel arn_norm(args) would launch on a device with `compute_units` CUs:
 * it runs arn_norm's argument checks and shape choice (the calling thread's
 * forced tile included) and copies into buf (size len, NUL-terminated,
 * truncated to fit; 160 bytes always suffice) the description arn_last_plan
 * would give after that call, with grid = the blocks of its last launch.
 * The pointers in args are only compared and their alignment read; nothing
 * is dereferenced.  Returns the status arn_norm would return before
 * launching (buf is left empty unless ARN_OK with rows > 0); ARN_EINVAL for
 * compute_units <= 0.  (struct arn_norm_args is declared in arn.h.)
 */
struct arn_norm_args;
int arn_norm_plan(const struct arn_norm_args *args, int compute_units, char *buf, size_t len);

#ifdef __cplusplus
}
#endif

#endif /* ARN_TUNING_H */
