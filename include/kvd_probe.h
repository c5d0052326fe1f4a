/*
 * kvd_probe.h -- a measurement helper exported by libkvd.so beside the decode
 * path (include/kvd.h).  It is not a step of the decode step and the pages
 * define no such operation: it reads a buffer as fast as a plain kernel of a
 * given grid shape can, which gives the practical ceiling against which the
 * decode kernels' achieved HBM bandwidth is reported (beside the fraction of
 * the device's 8 TB/s peak).
 */
#ifndef KVD_PROBE_H
#define KVD_PROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Read `bytes` of device memory at `buf` once, asynchronously on `stream`:
 * `workgroups` workgroups of `threads` threads each read a contiguous share,
 * 16 bytes per lane per load with `unroll` loads in flight per lane.
 *
 *   buf      device pointer, 16-byte aligned; bytes a multiple of 16.
 *   workgroups  1 .. 2^20;  threads  64 .. 1024, a multiple of 64;
 *   unroll   1, 2, 4, 8 or 16.
 *   sink     device pointer to one 32-bit word, written only in the rare
 *            case that the data folds to a fixed pattern (it keeps the
 *            loads alive).
 * Returns 0 on success, 1 for a NULL pointer, 2 for a bad size or
 * alignment, 3 for an unsupported unroll, 5 if the launch failed.  The
 * caller times the call (HIP events on the same stream).
 */
int32_t kvd_probe_stream_read(const void *buf, size_t bytes, int32_t workgroups, int32_t threads,
                              int32_t unroll, void *sink, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* KVD_PROBE_H */
