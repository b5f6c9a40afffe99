/*
 * tdi8_ceilings.h -- roofline calibration kernels (libtdi8_ceilings.so), a
 * measurement aid beside the GEMM library, used by bench.py --ceilings.
 *
 * The roofline the pages set out ("CUDA编程实践", section 3: compare a
 * kernel's compute intensity with peak compute over memory bandwidth) is
 * drawn here with the vendor's published peaks; these kernels measure what
 * the same hardware reaches in practice for the operations the GEMM kernels
 * are made of, so a kernel's distance from its roofline can be split into
 * what the hardware allows and what the kernel loses.
 *
 * All pointers are device memory owned by the caller; every call is
 * asynchronous on `stream` and returns 0, -1 (NULL pointer), -2 (invalid
 * size) or -(hipError_t) of a failed launch.  `cycles` receives one 64-bit
 * shader-clock count per block (s_memtime around the timed loop).
 */
#ifndef TDI8_CEILINGS_H
#define TDI8_CEILINGS_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t *hipStream_t;

/* v_mfma_i32_32x32x32_i8 back to back, eight independent accumulators per
 * wave, blocks of 256 threads (one wave per SIMD when one block per compute
 * unit runs).  operands: 16 * 256 16-byte values (64 KiB) read once into
 * registers; iters rounds of 8 instructions per wave; out: blocks * 256 int32
 * (results, so the work is kept); cycles: blocks entries.  Work per call:
 * blocks * 4 * iters * 8 * 65536 int8 operations. */
int tdi8c_mfma_loop(const int8_t *operands, int blocks, int iters, int32_t *out, uint64_t *cycles,
                    hipStream_t stream);

/* Read `bytes` (a multiple of 16) at src with 16-byte loads, `blocks` blocks
 * of 256 threads; out: one int32 (written only for an improbable value). */
int tdi8c_stream_read(const int8_t *src, int64_t bytes, int blocks, int32_t *out, hipStream_t stream);

/* Move `bytes` at src into LDS with global_load_lds_dwordx4: block b takes
 * the contiguous slab [b s, (b + 1) s), s = bytes / blocks (a multiple of
 * 1 KiB, at most 64 KiB), in 1 KiB wave pieces, every load issued before one
 * wait; threads a multiple of 64 up to 1024; nontemporal != 0 sets the
 * non-temporal cache policy on the loads (the skinny kernel's B stream).
 * out: one int32 (written only for an improbable value). */
int tdi8c_dma_read(const int8_t *src, int64_t bytes, int blocks, int threads, int nontemporal, int32_t *out,
                   hipStream_t stream);

/* 16-byte loads at region + misalign + 16 c over a 1 MiB region (c < 65536;
 * the caller provides 1 MiB + 16 bytes), blocks of 512 threads, iters rounds
 * of eight loads per lane; out: 512 int32; cycles: blocks entries.  Bytes
 * read per call: blocks * 512 * 16 * 8 * iters. */
int tdi8c_load16(const int8_t *region, int misalign, int blocks, int iters, int32_t *out, uint64_t *cycles,
                 hipStream_t stream);

/* A grid of blocks x threads that does nothing. */
int tdi8c_empty(int blocks, int threads, hipStream_t stream);

/* One K tile of the 256 x 256 GEMM configuration's loop, iters times, in
 * `blocks` blocks of 512 threads (8 waves): per wave and K step eight
 * v_mfma_i32_32x32x32_i8 on operands from six ds_read_b128 (the next step's
 * reads issued before this step's instructions), per K tile 64 KiB moved
 * into the other half of the 128 KiB LDS by global_load_lds_dwordx4 from a
 * 64 KiB window of src, then a barrier.  mode: bit 0 the LDS reads, bit 1
 * the DMA, bit 2 the matrix instructions (a part switched off is left out;
 * without reads the instructions take register operands).  src: at least
 * 1 MiB (the LDS starts as a copy of its first 128 KiB, so the operands
 * are src's bytes); out: 512 int32; cycles: blocks entries.  Per block and
 * iteration: 256 instructions (16.8 M int8 operations), 192 KiB of LDS
 * reads, 64 KiB of DMA. */
int tdi8c_loop_mix(const int8_t *src, int mode, int blocks, int iters, int32_t *out, uint64_t *cycles,
                   hipStream_t stream);

/* Write tiles_m x tiles_n tiles of 256 x 256 int32 (row stride ldc
 * elements, at least 256 tiles_n) at C, one block of 512 threads per tile
 * in the GEMM's XCD-grouped tile order, with non-temporal 16-byte stores of
 * whole rows (the 256 x 256 kernel's epilogue without its matrix work).
 * seed: the values written. */
int tdi8c_store_tiles(int32_t *C, int tiles_m, int tiles_n, int64_t ldc, int seed, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* TDI8_CEILINGS_H */
