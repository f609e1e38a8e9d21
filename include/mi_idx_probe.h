/*
 * mi_idx_probe.h -- HBM read and matrix-core ceilings of one MI355X
 * (libmi_idx_probe.so).
 *
 * Measurement aids, not part of the indexer: the pages define no such
 * operation.  The benchmark times them next to the two phases, so that the
 * decode's bandwidth is reported against both the 8 TB/s specification
 * figure and what a plain read of HBM reaches on the same GPU, and the
 * prefill's contraction against both the dense MFMA specification figure
 * and what the exact MFMA instruction it issues reaches.  Conventions as in
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

/* The device's compute-unit count, its shader clock and the constant
 * wall-clock counter's rate, in kHz, as the runtime reports them. */
int mi_idx_probe_device(int *cus, int *clock_khz, int *wall_clock_khz);

/* blocks_per_cu (1..8) workgroups of 256 threads per compute unit, each wave
 * issuing `iters` x 8 MFMAs of one instruction:
 *   kind 0  v_mfma_scale_f32_16x16x128_f8f6f4, A FP4 E2M1 (E8M0 scale),
 *           B FP8 E4M3 -- the prefill scorer's instruction, 65 536 flops;
 *   kind 1  v_mfma_f32_16x16x32_bf16 -- its bfloat16-query form, 16 384.
 * fold 0: 8 independent accumulating chains (the instruction's rate);
 * fold 1: the scorer's pattern -- a zeroed accumulator each time, its four
 * outputs folded into a running maximum with max3.  a_word / b_word fill
 * the operand registers (pick small values, e.g. 0x22222222 and 0x38383838,
 * so the chains stay finite; the rate does not depend on them).
 * sink: >= 256 * blocks_per_cu * CUs uint32 words, practically never written.
 * clocks[0] / clocks[1]: the shader-clock and wall-clock ticks workgroup 0's
 * first wave spent in its loop (clocks: 2 device uint64). */
int mi_idx_probe_mfma(int kind, int fold, int iters, int blocks_per_cu, uint32_t a_word,
                      uint32_t b_word, uint32_t *sink, int64_t sink_words, uint64_t *clocks,
                      void *stream);

#ifdef __cplusplus
}
#endif

#endif /* MI_IDX_PROBE_H */
