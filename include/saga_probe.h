/*
 * saga_probe.h -- C ABI of libsaga_probe.so, the HBM measurement kernels that
 * calibrate the decode library's roofline on MI355X (gfx950).
 *
 * Not part of the decode path: these kernels move bytes in the two access
 * patterns the decode step is made of, so that the step's achieved bandwidth
 * can be set against what this GPU sustains for the same pattern, next to the
 * published 8 TB/s peak:
 *   - a sequential read of contiguous chunks, one per workgroup (the pattern
 *     of the K stream, which reads every key row once);
 *   - a read of randomly placed rows of 64, 128 or 256 bytes (the pattern of
 *     the sparse value gather, which reads only the selected value rows).
 * Every value loaded is folded into one 32-bit word per workgroup, written to
 * sink_dev[workgroup], so no load can be dropped.
 *
 * Conventions: device pointers, 256-byte aligned; work is enqueued on
 * `stream` (a hipStream_t; NULL = the legacy default stream); nothing is
 * allocated, copied or synchronised.  Return 0 on success, 1 for an invalid
 * argument (null pointer, misalignment, a size or count out of range), 4 if a
 * launch failed.
 */
#ifndef SAGA_PROBE_H
#define SAGA_PROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Sequential read of buf_dev[0 .. bytes): workgroup w of `workgroups`
 * (1 .. 65535) reads the w-th of `workgroups` equal contiguous chunks with
 * 16-byte loads, `depth` (1, 2, 4 or 8) loads in flight per lane.  bytes is a
 * multiple of workgroups * 4096 and below 2^40.  sink_dev: uint32
 * [workgroups]. */
int saga_probe_read(const void* buf_dev, size_t bytes, int32_t workgroups, int32_t depth,
                    uint32_t* sink_dev, void* stream);

/* The same sequential read in the K stream's lane mapping: the 4 waves of
 * each workgroup read 16-row tiles of row_bytes (128 or 256) bytes, lane l
 * loading 16 bytes of row l % 16 at bytes 16 * (l / 16) + 64 m for
 * m < row_bytes / 64, `tiles` (1 or 2) tiles per wave in each of two batches
 * in flight.  bytes is a multiple of workgroups * 16384 and below 2^40; the
 * chunk of a workgroup is below 2^31 bytes.  sink_dev: uint32 [workgroups]. */
int saga_probe_read_tiles(const void* buf_dev, size_t bytes, int32_t row_bytes,
                          int32_t workgroups, int32_t tiles, uint32_t* sink_dev, void* stream);

/* Random-row read: `rows` rows of row_bytes (64, 128 or 256) bytes each, from
 * the buf_bytes / row_bytes rows of buf_dev (buf_bytes a multiple of row_bytes,
 * below 2^40).  Row k of the launch is row hash(seed, k) mod (buf_bytes /
 * row_bytes), hash being a 32-bit integer mixing function, so another seed
 * reads other rows.  row_bytes / 16 lanes read one row; each lane keeps
 * `depth` (1, 2, 4 or 8) rows in flight; `workgroups` (1 .. 2^20) workgroups
 * of 256 threads share the rows.  sink_dev: uint32 [workgroups]. */
int saga_probe_rows(const void* buf_dev, size_t buf_bytes, int32_t row_bytes, int64_t rows,
                    uint32_t seed, int32_t workgroups, int32_t depth, uint32_t* sink_dev,
                    void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SAGA_PROBE_H */
