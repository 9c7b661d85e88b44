/*
 * arn_probe.h -- measurement aid, not part of the operator library: plain
 * streaming kernels (lib/libarn_probe.so) that give the HBM bandwidth a mix
 * of read and write streams reaches on this GPU.  An operator that moves
 * the same byte mix cannot stream faster, so this is the practical ceiling
 * its roofline fraction is read against, next to the published peak.
 */
#ifndef ARN_PROBE_H
#define ARN_PROBE_H

#include <stdint.h>
#include <hip/hip_runtime.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * One launch of a grid-stride streaming kernel over n elements (1 <= n <=
 * 2^27): `reads` (0..2) streams of 16 bytes per element are read from a
 * then b; `writes16` (0..2) streams of 16 bytes per element are written to c
 * then d, and `writes8` (0..1) stream of 8 bytes per element to d.  Served
 * mixes (reads, writes16, writes8): (1,0,0) (0,1,0) (1,1,0) (2,2,0) (2,1,1)
 * (2,0,1).  c must be valid for every mix (the read-only mix keeps a
 * never-taken store to it); a, b, c, d are device buffers of n x 16 bytes
 * (d: n x 8 for the 8-byte stream), 16-byte aligned.  grid in 1..2^24,
 * block 256, 512 or 1024 threads, asynchronous on `stream`.  Returns 0, or
 * 1 (invalid argument), 2 (mix not served), 3 (launch failed).
 */
int arn_probe_stream(int reads, int writes16, int writes8, const void *a, const void *b,
                     void *c, void *d, int64_t n, int grid, int block, hipStream_t stream);

/*
 * The same with many read streams: `reads` streams of 16 bytes per element
 * from the host array srcs (device pointers), summed and written as
 * `writes16` 16-byte streams (c, then d) and `writes8` 8-byte streams (d).
 * Served mixes: (9, 2, 0) -- eight all-reduce parts and the residual read,
 * residual and 16-bit output written -- and (9, 1, 1) with an e4m3 output.
 * c and d must be valid.  Returns as arn_probe_stream.
 */
int arn_probe_stream_many(int reads, int writes16, int writes8, const void *const *srcs,
                          void *c, void *d, int64_t n, int grid, int block,
                          hipStream_t stream);

/*
 * The fused norm's row traffic without its arithmetic: for `rows` rows of
 * row_bytes bytes (multiple of 16, at most 16384) at a pitch of
 * stride_bytes, read x and res, write res in place and out.  Each block of
 * 512 threads owns rows_per_block (1, 2 or 4) consecutive rows and orders
 * its accesses by `mode`: 0 row by row (load, store, store), 1 all loads
 * then each row's stores, 2 all loads then all residual stores then all
 * output stores, 3 the next row's loads before the current row's stores.
 * x, res, out: device buffers of (rows - 1) * stride_bytes + row_bytes
 * bytes.  Returns 0, 1 (invalid argument), 2 (rows_per_block not served)
 * or 3 (launch failed).
 */
int arn_probe_rows(int mode, int rows_per_block, const void *x, void *res, void *out,
                   int64_t rows, int64_t row_bytes, int64_t stride_bytes, hipStream_t stream);

/*
 * One launch of an empty kernel (grid 1..2^24 blocks of 1..1024 threads) on
 * `stream`: the launch cost that bounds the time per call of small kernels
 * from below.  Returns 0, 1 (invalid argument) or 3 (launch failed).
 */
int arn_probe_empty(int grid, int block, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* ARN_PROBE_H */
