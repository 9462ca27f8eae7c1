/*
 * splitkv_probe.h -- measurement aids exported by libsplitkv.so.
 *
 * Not part of the attention operation. The benchmark uses them to measure the
 * denominator of its bandwidth figures and to evict the 256 MB Infinity Cache
 * between timed replays; the traffic counters are scaled by a plain copy of
 * known size. Same conventions as splitkv.h: device pointers owned by the
 * caller, work only enqueued on `stream`, host-side validation first,
 * negative status on error (codes of splitkv.h).
 */
#ifndef SPLITKV_PROBE_H
#define SPLITKV_PROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Streams `bytes` of `buf` through 16-byte loads and folds them into one
 * word per workgroup (written to `sink` only under a condition the data never
 * meets, so the loads cannot be dropped). buf 16-byte aligned, bytes a
 * multiple of 16; sink holds `grid` uint32 words. grid = number of
 * workgroups (256 threads each), 1..1048576. Used as the HBM read-peak probe
 * and, over a buffer larger than the Infinity Cache, as the cache flush. */
int splitkv_probe_read(const void *buf, size_t bytes, uint32_t *sink,
                       int grid, void *stream);

/* Copies `bytes` from src to dst with 16-byte loads and stores (both 16-byte
 * aligned, bytes a multiple of 16, no overlap). The known-size kernel that
 * scales the HBM traffic counters. */
int splitkv_probe_copy(const void *src, void *dst, size_t bytes, int grid,
                       void *stream);

#ifdef __cplusplus
}
#endif

#endif /* SPLITKV_PROBE_H */
