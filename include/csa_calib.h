/*
 * csa_calib.h -- calibration kernels for measuring what one MI355X (gfx950)
 * achieves, beside its datasheet peaks.  Measurement infrastructure used by
 * bench.py, not part of the indexer: the indexer's entry points are in
 * csa_index.h.
 *
 * All pointers are device pointers owned by the caller; work is enqueued on
 * `stream` (a hipStream_t) and nothing is synchronised or allocated.  Each
 * function returns 0 on success, or the HIP error code of the launch.
 */
#ifndef CSA_CALIB_H
#define CSA_CALIB_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Dense bf16 matrix-core loop: `blocks` workgroups of 256 threads, each wave
 * running `iters` rounds of 8 back-to-back v_mfma_f32_32x32x16_bf16 on four
 * independent accumulators, operands held in registers and taken from
 * `operands` (at least 256 * 16 bytes of bf16 values: their bit patterns set
 * the switching activity, e.g. Gaussian values or zeros).  Each wave writes
 * one float of its accumulators to sink[global wave id] so nothing is
 * optimised away (sink: blocks * 4 floats).  Flops per call:
 * blocks * 4 waves * iters * 8 * 32768.
 */
int32_t csa_calib_mfma_bf16(const void *operands, float *sink, int32_t blocks, int32_t iters, void *stream);

/*
 * Streaming read of `bytes` bytes (a multiple of 16) at `src` by `blocks`
 * workgroups of 256 threads with 16-byte loads, grid-stride, eight loads in
 * flight per thread; each thread adds what it reads and writes one word to
 * sink[thread id] (sink: blocks * 256 words).
 */
int32_t csa_calib_read(const void *src, size_t bytes, uint32_t *sink, int32_t blocks, void *stream);

/* Copy of `bytes` bytes (a multiple of 16) from src to dst with 16-byte loads
 * and stores, grid-stride over `blocks` workgroups of 256 threads. */
int32_t csa_calib_copy(const void *src, void *dst, size_t bytes, int32_t blocks, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* CSA_CALIB_H */
