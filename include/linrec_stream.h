/*
 * linrec_stream.h -- C ABI of libstream_ceiling.so, the streaming ceiling that
 * the scan's throughput is measured against.  It is not part of the scan
 * library and computes nothing of the recurrence.
 *
 * The scan moves 12 bytes per fp32 element: it reads a and b and writes h, and
 * nothing else counts (the traffic estimate of the first reasoning block of
 * the POPCORNBENCH "Kimi-K2.6 l1_p9" transcript: three tensors of B*L*D floats,
 * about 402 MB at B=32 L=4096 D=256).  The fastest any kernel can move those
 * bytes on a part is bounded by how fast a plain read-two-write-one stream
 * moves them there, so this library provides exactly that stream:
 *
 *     z[i] = x[i] + y[i]        i = 0 .. n-1
 *
 * with the scan kernel's memory instructions (128-bit nontemporal buffer loads
 * and stores), and lets the caller walk the arrays either contiguously or in
 * the scan's order over batch rows.
 */
#ifndef LINREC_STREAM_H
#define LINREC_STREAM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * linrec_stream_r2w1 -- enqueue z = x + y over n fp32 elements on `stream`.
 *
 *   x, y       input device buffers of n floats; z output device buffer of n
 *              floats (z must not overlap x or y).  All three 16-byte aligned.
 *   n          element count, a multiple of 4 * 64 * unroll (>= 0; 0 is a no-op).
 *   rows       1: walk the arrays contiguously.  R > 1: the arrays are R equal
 *              rows (n a multiple of R * 256 * unroll) and consecutive wave
 *              segments go to consecutive rows, the order in which the scan's
 *              persistent workgroups take one chunk of every batch row before
 *              the next chunk.
 *   unroll     128-bit accesses per lane per segment: 1, 2 or 4 (segments of
 *              1, 2 or 4 KiB of each array per wave).
 *   groups_per_cu  persistent 256-thread workgroups per compute unit (1..16).
 *   stream     hipStream_t, or NULL for the null stream.
 *
 * Returns 0 when enqueued, 1 for invalid arguments, 2 for a HIP error (the
 * text is in linrec_stream_last_error()).  Nothing is allocated.
 */
int linrec_stream_r2w1(const float *x, const float *y, float *z, int64_t n, int64_t rows, int32_t unroll,
                       int32_t groups_per_cu, void *stream);

/*
 * linrec_stream_column_walk -- enqueue z = x + y over three (B, L, D) fp32
 * arrays (contiguous, D fastest) in the walk of the scan's local-carry plans:
 * one workgroup per (batch row, slab of 4 * lanes channels) sequence, `waves`
 * waves whose lanes each take 4 channels and `steps_per_lane` consecutive rows,
 * tiles of waves * (64 / lanes) * steps_per_lane rows taken in order along L
 * with the next tile's loads in flight, and two workgroup barriers per tile.
 *
 *   lanes            8, 16, 32 or 64 (slabs of 128, 256, 512 or 1024 bytes);
 *                    D a multiple of 4 * lanes.
 *   waves            1, 2, 4 or 8.
 *   steps_per_lane   4 or 8.
 *   (L + 512) * D * 4 bytes must stay below 2 GiB (one batch row of an array,
 *                    and the rows a tile reaches past its end).
 *   Buffers as for linrec_stream_r2w1 (16-byte aligned, z disjoint from x, y).
 *
 * Returns 0 when enqueued (also for an empty shape), 1 for invalid arguments,
 * 2 for a HIP error.  Nothing is allocated.
 */
int linrec_stream_column_walk(const float *x, const float *y, float *z, int64_t B, int64_t L, int64_t D,
                              int32_t lanes, int32_t waves, int32_t steps_per_lane, void *stream);

/* Text of the calling thread's last failure ("" if none). */
const char *linrec_stream_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* LINREC_STREAM_H */
