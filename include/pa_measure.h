/*
 * pa_measure.h -- measurement calls of the paged KV cache library (gfx950).
 *
 * These are not part of the method: they time the library's kernels and give
 * the device's practical read rate as a yardstick beside the spec peak.  A
 * user of the method needs only pa.h.  Conventions (status codes, device
 * pointers, asynchrony) are those of pa.h.
 */
#ifndef PA_MEASURE_H
#define PA_MEASURE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Kernel timing: the next partition pass of the calling host thread (that of
 * pa_decode, pa_decode_append, pa_decode_partitions or
 * pa_decode_append_partitions) records start_event when its first
 * partition-kernel dispatch starts and stop_event when its last one ends
 * (hipExtLaunchKernel's dispatch events, the same clock a kernel trace
 * reports); the request is then cleared.  A call that returns an error before
 * launching leaves it pending.  Events are hipEvent_t values the caller
 * created, on the call's device; either may be NULL (NULL and NULL clears a
 * pending request).  Same kernels, same results; such a launch costs a few
 * microseconds more than a plain one.  Returns PA_OK. */
int pa_time_next_partitions(void* start_event, void* stop_event);

/* A plain streaming read of one contiguous device buffer: the practical HBM
 * read rate of this device, the yardstick beside the spec peak for
 * pa_decode's rate (pa_decode reads the same kind of bytes, scattered over
 * blocks).  Not part of the attention path.
 *   src:           device, 16-byte aligned; bytes a multiple of 16.
 *   blocks_per_cu: workgroups (256 threads) per compute unit, 1..64; the
 *                  grid-stride loop covers any size.
 *   unroll:        independent 16-byte non-temporal loads per thread and loop
 *                  trip: 1, 4, 8 or 16 (PA_ERR_UNSUPPORTED otherwise).
 *   blocked:       0: grid-stride (each load of the grid covers one contiguous
 *                  band, 4 KB per workgroup); 1: each workgroup reads
 *                  unroll x 4 KB contiguous bytes per loop trip.
 *   sink:          device, 4 bytes, written only in the unlikely case that the
 *                  XOR of all words a thread read equals 0x9e3779b9.
 * PA_ERR_INVALID_ARG for a null pointer, misalignment, blocks_per_cu outside
 * 1..64 or blocked not 0 or 1.  Asynchronous on stream. */
int pa_stream_read(const void* src, size_t bytes, int32_t blocks_per_cu, int32_t unroll, int32_t blocked,
                   void* sink, void* stream);

/* The practical ceiling of the prefill's inner loop: the same instructions
 * per 64-key tile and wave as pa_prefill's loop (32 MFMA 32x32x16 bf16, each
 * with a conflict-free 16-byte LDS fragment read, one multiply-add and one
 * exp2, a bf16 pair conversion and a row-sum step per two) and the same tile
 * traffic (32 KB per workgroup and tile from global memory into the idle half
 * of a double-buffered LDS tile, one load per four MFMAs, a wait and a
 * barrier), two 4-wave workgroups per compute unit, with no paging or
 * masking, and the vector work free of the MFMAs' results (each exponential
 * is consumed four steps later, the row sums go to four accumulators) so
 * that the hardware overlaps the two as far as it can.  The yardstick beside
 * the spec MFMA peak for pa_prefill's rate.
 *   src:        device, 16-byte aligned, >= 2 MiB (the tile loads cycle over
 *               its first 2 MiB; contents do not matter).
 *   iters:      tiles per wave (>= 1).
 *   mode:       0: MFMAs and fragment reads only; 1: plus the softmax
 *               arithmetic; 2: plus the tile loads, wait and barrier (the
 *               prefill's shape).
 *   sink:       device, 4 bytes, written only in the unlikely case the result
 *               folds to a marker value.
 *   flops_out:  HOST int64: the MFMA flops of the launch, for rating its time.
 * PA_ERR_INVALID_ARG for a null pointer, misalignment, src_bytes < 2 MiB,
 * iters < 1 or mode outside 0..2.  Asynchronous on stream. */
int pa_attention_loop_peak(const void* src, size_t src_bytes, int32_t iters, int32_t mode, void* sink,
                           int64_t* flops_out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PA_MEASURE_H */
