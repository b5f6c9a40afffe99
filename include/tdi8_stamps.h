/*
 * tdi8_stamps.h -- block timelines from the instrumented build of the
 * library (libtdi8_stamps.so), a measurement aid beside libtdi8.so, used by
 * bench.py --stamps.
 *
 * libtdi8_stamps.so is compiled from the same sources as libtdi8.so with
 * TDI8_STAMPS defined.  It exports every function of tdi8.h with the same
 * behaviour; in addition, while a record buffer is set, each block of every
 * GEMM and convolution kernel it launches writes one record of eight 64-bit
 * words, at index b = blockIdx.x + blockIdx.y * gridDim.x when b < capacity:
 *
 *   [0] shader clock (s_memtime) when the block starts
 *   [1] shader clock when its K loop is done (0 for a block that did none)
 *   [2] shader clock when it ends
 *   [3] 100 MHz constant clock (s_memrealtime) when it starts
 *   [4] 100 MHz constant clock when it ends
 *   [5] XCC_ID << 32 | HW_ID (the compute unit that ran it; HW_ID in the
 *       gfx9 layout: CU_ID bits 8-11, SH_ID bit 12, SE_ID bits 13-15)
 *   [6] b
 *   [7] 0
 *
 * The clocks stay in scalar registers until the block ends, and lane 0
 * writes the record last, so nothing in the block waits on the record.
 * The GEMM library's own kernels carry none of this.  Kernels that the
 * calls launch besides the GEMM (the zero fill before a K split) write no
 * records.  A later launch overwrites the records of an earlier one.
 */
#ifndef TDI8_STAMPS_H
#define TDI8_STAMPS_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Set the record buffer: `records` is device memory of at least
 * 64 * capacity bytes owned by the caller, used by every later launch of
 * this process until the next call; capacity 0 (records may be NULL) stops
 * the records.  Returns 0, or -1 (TDI8_ERR_INVALID_VALUE) for a negative
 * capacity or a NULL buffer with capacity > 0.  Not thread-safe against
 * concurrent launches. */
int tdi8_stamps_set(uint64_t *records, int capacity);

#ifdef __cplusplus
}
#endif

#endif /* TDI8_STAMPS_H */
