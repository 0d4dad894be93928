/*
 * rd_ceiling.h -- bandwidth probes for measurement (librd_ceiling.so).
 *
 * Not part of the reduction library: bench.py uses them to report the
 * bandwidth a trivial kernel reaches on the GPU it runs on, beside the
 * reductions' fraction of the published 8 TB/s HBM peak of an MI355X.
 * They touch only the first floor(n/4)*4 floats (whole 16-byte chunks).
 *
 * rd_ceiling_read(x, n, blocks, sink, stream)
 *   x      device pointer to n floats, 16-byte aligned, n >= 4 (read only)
 *   blocks workgroups of 256 threads, 1 .. 2^20; grid-stride order
 *   sink   device pointer to blocks*256 floats, written (one per thread)
 * rd_ceiling_read_pieces(x, n, steps, sink, stream)
 *   x      as for rd_ceiling_read
 *   steps  1 .. 1024: workgroup b of 256 threads reads the chunks
 *          [b*P, (b+1)*P), P = steps*4096, 16 loads in flight per lane;
 *          ceil(n/4 / P) workgroups
 *   sink   device pointer to ceil(n/4 / P) floats, written (one per workgroup)
 * rd_ceiling_copy(x, y, n, blocks, stream)
 *   x, y   device pointers to n floats each, 16-byte aligned, disjoint;
 *          blocks as for rd_ceiling_read (grid-stride)
 * rd_ceiling_copy_flat(x, y, n, threads, stream)
 *   x, y   as for rd_ceiling_copy; one 16-byte chunk per thread, workgroups
 *          of `threads` (64, 256 or 1024), ceil(n/4 / threads) of them
 * Enqueued on `stream`; return 0 on success, 1 for an invalid argument
 * (nothing enqueued), 2 if the launch failed.  Caller-owned memory only.
 */
#ifndef RD_CEILING_H
#define RD_CEILING_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

int rd_ceiling_read(const float* x, int64_t n, int32_t blocks, float* sink, hipStream_t stream);
int rd_ceiling_read_pieces(const float* x, int64_t n, int32_t steps, float* sink,
                           hipStream_t stream);
int rd_ceiling_copy(const float* x, float* y, int64_t n, int32_t blocks, hipStream_t stream);
int rd_ceiling_copy_flat(const float* x, float* y, int64_t n, int32_t threads,
                         hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* RD_CEILING_H */
