/*
 * mi_idx_probe.h -- HBM read-ceiling probes of one MI355X (libmi_idx_probe.so).
 *
 * Measurement aids, not part of the indexer: the pages define no such
 * operation.  The benchmark times them next to the decode phase, so that its
 * bandwidth is reported against both the 8 TB/s specification figure and
 * what a plain read of HBM reaches on the same GPU.  Conventions as in
 * mi_idx.h: device pointers, asynchronous on `stream` (a hipStream_t as
 * void*), nothing allocated, no synchronization.  Each returns 0 on success,
 * 1 for a bad argument, 3 when `sink` is too small, 4 for a HIP error.
 */
#ifndef MI_IDX_PROBE_H
#define MI_IDX_PROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Reads the `bytes` bytes at `buf` (16-byte aligned; bytes rounded down to a
 * multiple of 16) once, as coalesced 16-byte loads: blocks_per_cu (1..64)
 * workgroups of 256 threads per compute unit take 32 KB chunks in turn, 8
 * loads per thread in flight.  sink: >= 256 * blocks_per_cu * CUs uint32
 * words of scratch the kernel practically never writes. */
int mi_idx_probe_read_stream(const void *buf, int64_t bytes, int blocks_per_cu,
                             uint32_t *sink, int64_t sink_words, void *stream);

/* Reads n_order whole 8704-byte pages of `pages` ([num_pages, 8704], 16-byte
 * aligned) in the order of `order` (int32 page ids; an id outside
 * [0, num_pages) is clamped into it): wave w reads entries
 * [w * per_wave, (w + 1) * per_wave) one page after another, all 544 chunks
 * of a page in flight at once and the next page issued before the current
 * one is consumed.  sink: >= 256 * ceil(waves / 4) words, waves =
 * ceil(n_order / per_wave). */
int mi_idx_probe_read_pages(const uint8_t *pages, int64_t num_pages,
                            const int32_t *order, int64_t n_order, int per_wave,
                            uint32_t *sink, int64_t sink_words, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* MI_IDX_PROBE_H */
