/* w4_probe.h - measurement probes for the MI355X (gfx950) W4 linear layer library.
 *
 * Not part of the layer and not in its C ABI (include/w4.h): a separate library,
 * libw4probe.so, that bench.py loads to measure the ceilings the layer's kernels are read
 * against.  Pointers are device pointers, the work is enqueued on `stream` (a hipStream_t,
 * NULL = default stream) and is asynchronous.  Return value: 0, 1 for an invalid argument
 * (nothing launched), 5 for a launch failure.
 */
#ifndef W4_PROBE_H
#define W4_PROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* `blocks` workgroups of 4 waves, each wave running `iters` rounds of four independent
 * v_mfma_i32_32x32x32_i8 (the GEMM's shape) on register operands that are pseudo-random
 * (random_operands != 0) or constant; one int32 checksum per lane goes to sink (blocks * 256
 * int32, 16-byte aligned).  Work: blocks * 4 * iters * 4 * 2 * 32^3 int ops.  Timing it gives
 * the sustained dense int8 MFMA rate with and without the datapath toggling that real
 * operands cause.  1 <= blocks <= 2^24, iters >= 1. */
int w4_probe_mfma_rate(int64_t blocks, int iters, int random_operands, int32_t *sink, void *stream);

/* Read `bytes` (a multiple of 16, 16-byte aligned src) once with `blocks` workgroups of 256
 * threads, 16-byte loads, eight in flight per thread; one int32 per thread to sink
 * (blocks * 256 int32, 16-byte aligned).  Timing it gives the HBM read rate a plain streaming
 * kernel reaches at that size: the practical ceiling of the HBM-bound small-M kernels.
 * 1 <= blocks <= 2^20. */
int w4_probe_read_rate(const void *src, int64_t bytes, int64_t blocks, int32_t *sink, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* W4_PROBE_H */
