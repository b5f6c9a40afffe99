// Device-side helpers shared by the gfx950 GEMM kernels: vector types,
// masked loads for the tail kernels, C stores.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

namespace tdi8 {

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x16 __attribute__((ext_vector_type(16)));

// Kernel arguments, passed by value.  Leading dimensions in elements.
struct GemmArgs {
    const int8_t *A;
    const int8_t *B;
    int32_t *C;
    int64_t lda, ldb, ldc;
    int M, N, K;
    int tiles_m, tiles_n;  // block tiles along M and N
    int splits;            // K slices (1: each block covers all of K)
#if defined(TDI8_STAMPS)
    uint64_t *stamps;      // timeline records (BlockStamp), one per block id below stamp_cap
    int stamp_cap;
#endif
};

// Convolution geometry (NHWC image, KRSC filters): image N x H x W x C,
// filters R x S, output P x Q, stride sh/sw, zero padding ph/pw, dilation
// dh/dw; rsc = R * S * C, the reduction length.  c_div and s_div divide
// reduction positions by C and by S without a division instruction.
struct FastDiv {
    unsigned magic;
    int shift;
};
struct ConvParams {
    int N, H, W, C, R, S, P, Q;
    int sh, sw, ph, pw, dh, dw;
    int rsc;
    FastDiv c_div, s_div;
    int tile_in_tap;  // C a multiple of the K tile: every K tile lies within one tap
    int run;          // gather form with dw = 1: S C, the bytes of a filter row (else 0), see conv_run16
    int runp;         // 16-byte pieces per filter row, ceil(S C / 16)
    FastDiv runp_div;
};

// Division by a divisor d >= 1 fixed for the whole launch, for 0 <= n < 2^31
// (Granlund and Montgomery, "Division by invariant integers using
// multiplication", 1994): with l = ceil(log2 d) and
// magic = floor(2^32 (2^l - d) / d) + 1, n / d = (mulhi(n, magic) + n) >> l.
// The sum stays below 2^32 because mulhi(n, magic) < n < 2^31.
inline FastDiv make_fast_div(int d) {
    int l = 0;
    while ((int64_t{1} << l) < d) ++l;
    const uint64_t m = ((uint64_t{1} << 32) * ((uint64_t{1} << l) - static_cast<uint64_t>(d))) /
                           static_cast<uint64_t>(d) + 1;
    return FastDiv{static_cast<unsigned>(m), l};
}
__device__ __forceinline__ int fast_div(int n, FastDiv f) {
    const unsigned nn = static_cast<unsigned>(n);
    return static_cast<int>((__umulhi(nn, f.magic) + nn) >> f.shift);
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt bits [3:0] and [15:14], expcnt [6:4] and lgkmcnt [11:8] left at max).
#define TDI8_WAIT_VMCNT(n) \
    __builtin_amdgcn_s_waitcnt(((n) & 0xF) | (0x7 << 4) | (0xF << 8) | ((((n) >> 4) & 3) << 14))
// s_waitcnt lgkmcnt(0) with the other counters left at max.
#define TDI8_WAIT_LGKM0() __builtin_amdgcn_s_waitcnt(0xF | (0x7 << 4) | (0x0 << 8) | (3 << 14))

// Block barrier that waits on no memory counter (callers first wait for
// exactly what they need; __syncthreads() also waits for every outstanding
// global load) and that the compiler may not move memory accesses across:
// the barrier builtin alone is not a memory operation to the optimiser, the
// empty asm statements with a memory clobber are.
__device__ __forceinline__ void block_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// f(std::integral_constant<int, I>{}) for I = 0 .. N-1 in order: loop bodies
// that index register arrays by a compile-time value.
template <class F, int... I>
__device__ __forceinline__ void static_for_impl(F &f, std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F &&f) {
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

__device__ __forceinline__ int clamp16(int v) { return v < 0 ? 0 : (v > 16 ? 16 : v); }
__device__ __forceinline__ int clamp4(int v) { return v < 0 ? 0 : (v > 4 ? 4 : v); }

// 16 bytes at p; p is 16-byte aligned (unpredicated kernels).
__device__ __forceinline__ i32x4 load16(const int8_t *p) {
    return *reinterpret_cast<const i32x4 *>(p);
}

// Keep the low `nvalid` bytes (0..4) of a dword.
__device__ __forceinline__ uint32_t keep_bytes(uint32_t w, int nvalid) {
    return nvalid >= 4 ? w : (nvalid <= 0 ? 0u : (w & ((1u << (8 * nvalid)) - 1u)));
}

// v with every byte moved up by n bytes (byte i to i + n, zeros below;
// 0 <= n < 16).
__device__ __forceinline__ i32x4 shift_up_bytes(i32x4 v, int n) {
    const uint64_t lo = static_cast<uint32_t>(v[0]) | (static_cast<uint64_t>(static_cast<uint32_t>(v[1])) << 32);
    const uint64_t hi = static_cast<uint32_t>(v[2]) | (static_cast<uint64_t>(static_cast<uint32_t>(v[3])) << 32);
    const int b = 8 * n;
    uint64_t nlo = 0, nhi = lo << (b >= 64 ? b - 64 : 0);
    if (b < 64) {
        nlo = lo << b;
        nhi = b == 0 ? hi : (hi << b) | (lo >> (64 - b));
    }
    return i32x4{static_cast<int32_t>(static_cast<uint32_t>(nlo)), static_cast<int32_t>(nlo >> 32),
                 static_cast<int32_t>(static_cast<uint32_t>(nhi)), static_cast<int32_t>(nhi >> 32)};
}

// v with every byte moved down by n bytes (byte i + n to i, zeros above;
// 0 <= n <= 16, so n = 16 gives zero).
__device__ __forceinline__ i32x4 shift_down_bytes(i32x4 v, int n) {
    const uint64_t lo = static_cast<uint32_t>(v[0]) | (static_cast<uint64_t>(static_cast<uint32_t>(v[1])) << 32);
    const uint64_t hi = static_cast<uint32_t>(v[2]) | (static_cast<uint64_t>(static_cast<uint32_t>(v[3])) << 32);
    const int b = 8 * n;
    const uint64_t nhi = b >= 64 ? 0 : hi >> b;
    const uint64_t nlo = b >= 128 ? 0 : b >= 64 ? hi >> (b - 64) : b == 0 ? lo : (lo >> b) | (hi << (64 - b));
    return i32x4{static_cast<int32_t>(static_cast<uint32_t>(nlo)), static_cast<int32_t>(nlo >> 32),
                 static_cast<int32_t>(static_cast<uint32_t>(nhi)), static_cast<int32_t>(nhi >> 32)};
}

// 16 bytes at p, any alignment: one global_load_dwordx4 (the ROCm driver
// runs gfx9-class GPUs in unaligned-access mode, and the compiler lowers an
// unaligned 16-byte copy to exactly this instruction).
__device__ __forceinline__ i32x4 load16_unaligned(const int8_t *p) {
    i32x4 v;
    __builtin_memcpy(&v, p, 16);
    return v;
}

// The first `nvalid` (0..16) bytes at p, any alignment, zero beyond.  A full
// chunk is one load; for a partial chunk only dwords holding at least one
// wanted byte are read (an aligned dword never straddles a page, so nothing
// outside the operand's pages is touched).
__device__ __forceinline__ i32x4 load16_masked(const int8_t *p, int nvalid) {
    i32x4 r = {0, 0, 0, 0};
    if (nvalid <= 0) return r;
    const uintptr_t a = reinterpret_cast<uintptr_t>(p);
    if (nvalid >= 16) return load16_unaligned(p);
    const uint32_t s = static_cast<uint32_t>(a & 3);
    const uint32_t *w = reinterpret_cast<const uint32_t *>(a - s);
    uint32_t d[5];
#pragma unroll
    for (int i = 0; i < 5; ++i) d[i] = (4 * i < static_cast<int>(s) + nvalid) ? w[i] : 0u;
#pragma unroll
    for (int j = 0; j < 4; ++j)
        r[j] = static_cast<int32_t>(keep_bytes(__builtin_amdgcn_alignbyte(d[j + 1], d[j], s), nvalid - 4 * j));
    return r;
}

// The first `nvalid` (0..4) bytes at p, any alignment, zero beyond.
__device__ __forceinline__ uint32_t load4_masked(const int8_t *p, int nvalid) {
    if (nvalid <= 0) return 0u;
    const uintptr_t a = reinterpret_cast<uintptr_t>(p);
    if (nvalid >= 4) {
        uint32_t v;
        __builtin_memcpy(&v, p, 4);
        return v;
    }
    const uint32_t s = static_cast<uint32_t>(a & 3);
    const uint32_t *w = reinterpret_cast<const uint32_t *>(a - s);
    const uint32_t d0 = w[0];
    const uint32_t d1 = (4 < static_cast<int>(s) + nvalid) ? w[1] : 0u;
    return keep_bytes(__builtin_amdgcn_alignbyte(d1, d0, s), nvalid);
}

// 4x4 byte transpose: in[r] holds bytes (r,0..3); out[c] gets bytes (0..3,c).
__device__ __forceinline__ void transpose4x4(const uint32_t in[4], uint32_t out[4]) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const int sh = 8 * c;
        out[c] = ((in[0] >> sh) & 0xFFu) | (((in[1] >> sh) & 0xFFu) << 8) |
                 (((in[2] >> sh) & 0xFFu) << 16) | (((in[3] >> sh) & 0xFFu) << 24);
    }
}

// Four consecutive C elements of row m starting at column n.
template <bool FAST>
__device__ __forceinline__ void store4(const GemmArgs &g, int m, int n, i32x4 v) {
    if (FAST) {
        *reinterpret_cast<i32x4 *>(g.C + static_cast<int64_t>(m) * g.ldc + n) = v;
        return;
    }
    if (m >= g.M) return;
    int32_t *p = g.C + static_cast<int64_t>(m) * g.ldc + n;
    if (n + 3 < g.N) {
        __builtin_memcpy(p, &v, 16);  // one global_store_dwordx4, 4-byte aligned
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (n + e < g.N) p[e] = v[e];
    }
}

// Cache-policy operand of the LDS DMA load: the non-temporal hint, for a
// stream read once (B when a single block row covers M), so that it does not
// evict the lines the kernel reads again (A).
constexpr int kLoadStream = 2;

// store4 with the non-temporal hint, for epilogues whose store instructions
// write whole 128-byte lines of C (the C-through-LDS epilogues): C is not
// read again by the kernel, and hinted lines do not evict operand lines
// other blocks still use.  Four columns in range: one hinted 16-byte store
// (C need only be 4-byte aligned); the ragged edge goes through store4.
template <bool FAST>
__device__ __forceinline__ void store4_nt(const GemmArgs &g, int m, int n, i32x4 v) {
    typedef i32x4 i32x4_a4 __attribute__((aligned(4)));
    if (!FAST) {
        if (m >= g.M) return;
        if (n + 3 >= g.N) {
            store4<false>(g, m, n, v);
            return;
        }
    }
    __builtin_nontemporal_store(v, reinterpret_cast<i32x4_a4 *>(g.C + static_cast<int64_t>(m) * g.ldc + n));
}

// Block timeline, compiled only into the instrumented library
// (libtdi8_stamps.so, built with -DTDI8_STAMPS; the GEMM library's kernels do
// not contain it).  Per block: the shader clock (s_memtime) at entry, when
// the K loop is done and at exit, the constant 100 MHz clock (s_memrealtime)
// at entry and exit, and the hardware ids (HW_ID, XCC_ID) of the compute
// unit that ran it.  The clocks sit in scalar registers until the block
// ends; lane 0 of the block then writes one 64-byte record with vector
// stores, so nothing inside the timed stretch waits on memory for them.
struct BlockStamp {
#if defined(TDI8_STAMPS) && defined(__HIP_DEVICE_COMPILE__)
    uint64_t c0 = 0, cm = 0, r0 = 0;
    __device__ __forceinline__ void begin() {
        c0 = __builtin_amdgcn_s_memtime();
        r0 = __builtin_amdgcn_s_memrealtime();
    }
    __device__ __forceinline__ void loop_done() { cm = __builtin_amdgcn_s_memtime(); }
    __device__ __forceinline__ void end(const GemmArgs &g) {
        const uint64_t c1 = __builtin_amdgcn_s_memtime();
        const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
        uint32_t hw, xcc;
        asm volatile("s_getreg_b32 %0, hwreg(HW_REG_HW_ID)" : "=s"(hw));
        asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
        const int64_t b = blockIdx.x + static_cast<int64_t>(blockIdx.y) * gridDim.x;
        if (threadIdx.x == 0 && g.stamps != nullptr && b < g.stamp_cap) {
            uint64_t *r = g.stamps + 8 * b;
            r[0] = c0;
            r[1] = cm;
            r[2] = c1;
            r[3] = r0;
            r[4] = r1;
            r[5] = (static_cast<uint64_t>(xcc) << 32) | hw;
            r[6] = static_cast<uint64_t>(b);
            r[7] = 0;
        }
    }
#else
    __device__ __forceinline__ void begin() {}
    __device__ __forceinline__ void loop_done() {}
    __device__ __forceinline__ void end(const GemmArgs &) {}
#endif
};

}  // namespace tdi8
