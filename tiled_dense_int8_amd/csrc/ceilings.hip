// Roofline calibration kernels for gfx950 (measurement only; the GEMM
// library does not use them).  Each measures one practical ceiling that the
// GEMM kernels' roofline fractions are read against:
//  * tdi8c_mfma_loop: v_mfma_i32_32x32x32_i8 back to back on register
//    operands taken from a caller buffer, eight independent accumulators per
//    wave, one wave per SIMD: the matrix-core rate for those operand bytes
//    (random bytes switch more transistors than constant ones, and the clock
//    follows the power drawn);
//  * tdi8c_stream_read: a plain read of a buffer with 16-byte loads, the HBM
//    read rate a kernel of that size reaches;
//  * tdi8c_dma_read: the same bytes moved into LDS by global_load_lds_dwordx4
//    in per-block contiguous slabs, every load issued before the one wait
//    (the skinny kernel's B stream without its A, matrix work and epilogue);
//  * tdi8c_load16: 16-byte loads from a 1 MiB region that stays in L2, at a
//    given byte offset from 16-byte alignment (rows of a tight odd leading
//    dimension are misaligned);
//  * tdi8c_empty: a launch that does nothing, the fixed cost of a grid;
//  * tdi8c_loop_mix: the operations of one K tile of the 256 x 256 GEMM
//    configuration (per wave and K step eight v_mfma_i32_32x32x32_i8 fed by
//    six ds_read_b128, next step's reads issued first; per K tile 64 KiB
//    moved into LDS by DMA from an L2-resident source), with any of the
//    three parts switched off: the rate of each part alone and of the mix,
//    on the random bytes the LDS holds;
//  * tdi8c_store_tiles: 256 x 256 int32 tiles written by 512-thread blocks
//    in the GEMM's XCD-grouped tile order with the epilogue's whole-line
//    non-temporal stores: the C drain of the 256 x 256 kernel alone.
// Cycle counts come from s_memtime (the shader clock) per block.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "../../include/tdi8_ceilings.h"

namespace {

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x16 __attribute__((ext_vector_type(16)));
constexpr int kAcc = 8;

// 256 threads (one wave per SIMD); operands: 2 * kAcc * 256 16-byte values.
__global__ void __launch_bounds__(256) mfma_loop_kernel(const i32x4 *ops, int iters, int32_t *out,
                                                        uint64_t *cycles) {
    const int tid = threadIdx.x;
    i32x4 a[kAcc], b[kAcc];
#pragma unroll
    for (int j = 0; j < kAcc; ++j) {
        a[j] = ops[(2 * j) * 256 + tid];
        b[j] = ops[(2 * j + 1) * 256 + tid];
    }
    i32x16 acc[kAcc];
#pragma unroll
    for (int j = 0; j < kAcc; ++j) acc[j] = i32x16{};
    const uint64_t t0 = __builtin_amdgcn_s_memtime();
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < kAcc; ++j)
            acc[j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[j], b[(j + 1) % kAcc], acc[j], 0, 0, 0);
    }
    const uint64_t t1 = __builtin_amdgcn_s_memtime();
    int32_t s = 0;
#pragma unroll
    for (int j = 0; j < kAcc; ++j) s ^= acc[j][0] ^ acc[j][7] ^ acc[j][15];
    out[blockIdx.x * 256 + tid] = s;
    if (tid == 0) cycles[blockIdx.x] = t1 - t0;
}

// Every thread reads 16-byte chunks i, i + stride, ... (four in flight).
__global__ void __launch_bounds__(256) stream_read_kernel(const i32x4 *src, int64_t chunks, int32_t *out) {
    const int64_t stride = static_cast<int64_t>(gridDim.x) * 256;
    i32x4 acc = {0, 0, 0, 0};
    int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    for (; i + 3 * stride < chunks; i += 4 * stride) {
        const i32x4 v0 = src[i], v1 = src[i + stride], v2 = src[i + 2 * stride], v3 = src[i + 3 * stride];
        acc ^= v0 ^ v1 ^ v2 ^ v3;
    }
    for (; i < chunks; i += stride) acc ^= src[i];
    // written only for one improbable value, so the loads are kept and
    // nothing is stored in practice
    if ((acc[0] ^ acc[1] ^ acc[2] ^ acc[3]) == 0x5bd1e995) out[0] = 1;
}

// 512 threads; lane reads 16 bytes at base + misalign + 16 c, c inside the
// 1 MiB region (65536 chunks), eight loads in flight per wave.
__global__ void __launch_bounds__(512) load16_kernel(const int8_t *base, int misalign, int iters, int32_t *out,
                                                     uint64_t *cycles) {
    typedef i32x4 i32x4_u __attribute__((aligned(1)));
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    i32x4 acc = {0, 0, 0, 0};
    const uint64_t t0 = __builtin_amdgcn_s_memtime();
    for (int it = 0; it < iters; ++it) {
        i32x4 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int c = (static_cast<int>(blockIdx.x) * 977 + lane + 64 * (wave * 8 + u) + it * 4096) & 65535;
            v[u] = *reinterpret_cast<const i32x4_u *>(base + misalign + 16 * static_cast<int64_t>(c));
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) acc ^= v[u];
    }
    const uint64_t t1 = __builtin_amdgcn_s_memtime();
    if ((acc[0] ^ acc[1] ^ acc[2] ^ acc[3]) == 0x5bd1e995) out[tid] = 1;
    if (tid == 0) cycles[blockIdx.x] = t1 - t0;
}

// Block b moves bytes [b slab, (b + 1) slab) into LDS in 1 KiB wave pieces
// (slab a multiple of 1 KiB, at most 64 KiB); AUX: cache policy of the loads.
template <int AUX>
__global__ void __launch_bounds__(1024) dma_read_kernel(const int8_t *src, int64_t slab, int32_t *out) {
    __shared__ __attribute__((aligned(1024))) int8_t buf[65536];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
    const int8_t *p = src + static_cast<int64_t>(blockIdx.x) * slab;
    const int pieces = static_cast<int>(slab >> 10);
    for (int pc = wave; pc < pieces; pc += nw)
        __builtin_amdgcn_global_load_lds(p + pc * 1024 + lane * 16,
                                         (__attribute__((address_space(3))) void *)(buf + pc * 1024), 16, 0, AUX);
    __builtin_amdgcn_s_waitcnt(0 | (0x7 << 4) | (0xF << 8));  // vmcnt(0)
    __syncthreads();
    // written only for one improbable byte pattern, so the loads are kept
    const int t = (threadIdx.x * 16) & 65535;
    if (buf[t] == 0x7b && buf[t + 1] == 0x11 && buf[t + 2] == 0x13) out[0] = 1;
}

// One block of 512 threads (8 waves, two per SIMD) per compute unit.  The
// 128 KiB LDS starts as a copy of src (random bytes); MODE bit 0: operand
// reads, bit 1: DMA refills, bit 2: matrix instructions.  Iteration = one
// K tile: 4 steps x (6 reads + 8 instructions) per wave, 8 KiB of DMA per
// wave (64 KiB per block) into the other half of the LDS, then a barrier.
// src: at least 1 MiB; block b's DMA source is the 64 KiB window b mod 16.
template <int MODE>
__global__ void __launch_bounds__(512) loop_mix_kernel(const int8_t *src, int iters, int32_t *out, uint64_t *cycles) {
    __shared__ __attribute__((aligned(1024))) int8_t lds[128 * 1024];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    for (int i = tid; i < 128 * 1024 / 16; i += 512)
        reinterpret_cast<i32x4 *>(lds)[i] = reinterpret_cast<const i32x4 *>(src)[i];
    __syncthreads();
    i32x4 x = {0, 0, 0, 0};
    i32x16 acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = i32x16{};
    const int8_t *gsrc = src + (blockIdx.x % 16) * 65536;
    const uint64_t t0 = __builtin_amdgcn_s_memtime();
    for (int it = 0; it < iters; ++it) {
        const int stage = it & 1;
        i32x4 f[2][6];
        auto rd = [&](int s, int b) {
#pragma unroll
            for (int r = 0; r < 6; ++r) {
                if (MODE & 1)
                    f[b][r] = *reinterpret_cast<const i32x4 *>(lds + stage * 65536 + ((wave * 6 + r + s * 48) & 63) * 1024 +
                                                                lane * 16);
                else
                    f[b][r] = x + r + s;
            }
        };
        rd(0, 0);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int b = s & 1;
            if (s + 1 < 4) rd(s + 1, b ^ 1);
            if (MODE & 2) {
#pragma unroll
                for (int d = 0; d < 2; ++d) {
                    const int piece = (wave * 8 + s * 2 + d) & 63;
                    __builtin_amdgcn_global_load_lds(gsrc + piece * 1024 + lane * 16,
                                                     (__attribute__((address_space(3))) void *)(lds + (stage ^ 1) * 65536 +
                                                                                                  piece * 1024),
                                                     16, 0, 0);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
            if (MODE & 4) {
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    acc[j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(f[b][j % 2 + 4], f[b][j / 2], acc[j], 0, 0, 0);
            } else {
#pragma unroll
                for (int r = 0; r < 6; ++r) x ^= f[b][r];
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    }
    const uint64_t t1 = __builtin_amdgcn_s_memtime();
    int32_t v = x[0] ^ x[1] ^ x[2] ^ x[3];
#pragma unroll
    for (int j = 0; j < 8; ++j) v ^= acc[j][0] ^ acc[j][15];
    if (v == 0x5bd1e995) out[tid] = v;  // improbable: keeps the work, stores nothing in practice
    if (tid == 0) cycles[blockIdx.x] = t1 - t0;
}

// Block b writes the 256 x 256 int32 tile that the GEMM's XCD-grouped order
// gives block b (32 blocks of one XCD on a group of 4 tile rows), 64
// consecutive 16-byte pieces of one row per wave instruction, with the
// non-temporal hint, as the 256 x 256 kernel's epilogue does.
__global__ void __launch_bounds__(512) store_tiles_kernel(int32_t *C, int tiles_m, int tiles_n, int64_t ldc, int32_t seed) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int total = tiles_m * tiles_n;
    const int bid = blockIdx.x;
    int l = bid;
    if ((total & 7) == 0) l = (bid & 7) * (total >> 3) + (bid >> 3);
    const int gsize = 4 * tiles_n;
    const int first = (l / gsize) * 4;
    const int rows = min(tiles_m - first, 4);
    const int within = l % gsize;
    const int tm = first + within % rows, tn = within / rows;
    const i32x4 v = {seed + tid, seed ^ tid, 3 * tid, seed};
    for (int i = 0; i < 32; ++i) {
        const int r = wave + 8 * i;
        __builtin_nontemporal_store(v + i, reinterpret_cast<i32x4 *>(C + (static_cast<int64_t>(tm) * 256 + r) * ldc +
                                                                     tn * 256 + 4 * lane));
    }
}

__global__ void empty_kernel() {}

int status_of(hipError_t e) { return e == hipSuccess ? 0 : -static_cast<int>(e); }

}  // namespace

extern "C" {

int tdi8c_mfma_loop(const int8_t *operands, int blocks, int iters, int32_t *out, uint64_t *cycles,
                    hipStream_t stream) {
    if (!operands || !out || !cycles) return -1;
    if (blocks <= 0 || iters <= 0) return -2;
    hipLaunchKernelGGL(mfma_loop_kernel, dim3(blocks), dim3(256), 0, stream,
                       reinterpret_cast<const i32x4 *>(operands), iters, out, cycles);
    return status_of(hipGetLastError());
}

int tdi8c_stream_read(const int8_t *src, int64_t bytes, int blocks, int32_t *out, hipStream_t stream) {
    if (!src || !out) return -1;
    if (bytes < 16 || bytes % 16 != 0 || blocks <= 0) return -2;
    hipLaunchKernelGGL(stream_read_kernel, dim3(blocks), dim3(256), 0, stream, reinterpret_cast<const i32x4 *>(src),
                       bytes / 16, out);
    return status_of(hipGetLastError());
}

int tdi8c_dma_read(const int8_t *src, int64_t bytes, int blocks, int threads, int nontemporal, int32_t *out,
                   hipStream_t stream) {
    if (!src || !out) return -1;
    if (blocks <= 0 || threads < 64 || threads > 1024 || threads % 64 != 0 || bytes <= 0 || bytes % blocks != 0)
        return -2;
    const int64_t slab = bytes / blocks;
    if (slab % 1024 != 0 || slab > 65536) return -2;
    if (nontemporal)
        hipLaunchKernelGGL(dma_read_kernel<2>, dim3(blocks), dim3(threads), 0, stream, src, slab, out);
    else
        hipLaunchKernelGGL(dma_read_kernel<0>, dim3(blocks), dim3(threads), 0, stream, src, slab, out);
    return status_of(hipGetLastError());
}

int tdi8c_load16(const int8_t *region, int misalign, int blocks, int iters, int32_t *out, uint64_t *cycles,
                 hipStream_t stream) {
    if (!region || !out || !cycles) return -1;
    if (misalign < 0 || misalign > 15 || blocks <= 0 || iters <= 0) return -2;
    hipLaunchKernelGGL(load16_kernel, dim3(blocks), dim3(512), 0, stream, region, misalign, iters, out, cycles);
    return status_of(hipGetLastError());
}

int tdi8c_empty(int blocks, int threads, hipStream_t stream) {
    if (blocks <= 0 || threads <= 0 || threads > 1024) return -2;
    hipLaunchKernelGGL(empty_kernel, dim3(blocks), dim3(threads), 0, stream);
    return status_of(hipGetLastError());
}


int tdi8c_loop_mix(const int8_t *src, int mode, int blocks, int iters, int32_t *out, uint64_t *cycles,
                   hipStream_t stream) {
    if (!src || !out || !cycles) return -1;
    if (mode < 0 || mode > 7 || blocks <= 0 || iters <= 0) return -2;
    const dim3 g(blocks), b(512);
    switch (mode) {
    case 0: hipLaunchKernelGGL(loop_mix_kernel<0>, g, b, 0, stream, src, iters, out, cycles); break;
    case 1: hipLaunchKernelGGL(loop_mix_kernel<1>, g, b, 0, stream, src, iters, out, cycles); break;
    case 2: hipLaunchKernelGGL(loop_mix_kernel<2>, g, b, 0, stream, src, iters, out, cycles); break;
    case 3: hipLaunchKernelGGL(loop_mix_kernel<3>, g, b, 0, stream, src, iters, out, cycles); break;
    case 4: hipLaunchKernelGGL(loop_mix_kernel<4>, g, b, 0, stream, src, iters, out, cycles); break;
    case 5: hipLaunchKernelGGL(loop_mix_kernel<5>, g, b, 0, stream, src, iters, out, cycles); break;
    case 6: hipLaunchKernelGGL(loop_mix_kernel<6>, g, b, 0, stream, src, iters, out, cycles); break;
    default: hipLaunchKernelGGL(loop_mix_kernel<7>, g, b, 0, stream, src, iters, out, cycles); break;
    }
    return status_of(hipGetLastError());
}

int tdi8c_store_tiles(int32_t *C, int tiles_m, int tiles_n, int64_t ldc, int seed, hipStream_t stream) {
    if (!C) return -1;
    if (tiles_m <= 0 || tiles_n <= 0 || ldc < static_cast<int64_t>(tiles_n) * 256) return -2;
    hipLaunchKernelGGL(store_tiles_kernel, dim3(tiles_m * tiles_n), dim3(512), 0, stream, C, tiles_m, tiles_n, ldc,
                       seed);
    return status_of(hipGetLastError());
}

}  // extern "C"
