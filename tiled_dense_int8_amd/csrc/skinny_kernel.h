// Skinny-M int8 GEMM kernel for gfx950: the route taken when the fill step
// of the selection finds no tiling that gives every compute unit a block and
// M is small (patent application CN114238853A, claim 4, the "too small to
// fill the compute resources, reuse 1" branch).
//
// With M <= 32 the product is a stream over B: B is read from HBM exactly
// once and A (at most 32 rows) stays in L2.  Too few (M, N) tiles leave the
// latency of that stream unhidden (the contest write-up's "线程束调度空间受限"
// point: warps split only by (M, N) are not enough), so each block also
// splits K across its WK waves and reduces their int32 partial sums in LDS
// (exact in any order).
//
// Block: rows [m0, m0 + 16*MT), columns [n0, n0 + 16*NT), all of K.  Wave w
// takes K super-steps s = w, w + WK, ... of 256 bytes; in a super-step lane
// (r = lane % 16, g = lane / 16) loads 64 contiguous bytes of its B column
// and of its A row at k = 256*s + 64*g .. +63 and issues four
// v_mfma_i32_16x16x64_i8, the q-th taking bytes 16q..16q+15 of every lane.
// The K assignment is a permutation of K that A and B share, so each
// instruction pairs A(m, k) with B(k, n) for the same k.
//
// gemm_skinny_kernel takes column-major B (K-contiguous columns).  FAST:
// M % (16 MT) == 0, N % (16 NT) == 0, K % 256 == 0, 16-byte aligned A, B, C,
// lda and ldb multiples of 16, ldc of 4.
//
// gemm_skinny_rr_kernel takes row-major B (N contiguous).  There lane
// (r, g) reads, for the 16 rows k = 64*s + 16*g .. +15, the dword holding
// columns n0 + 4r .. +3, transposes the 16 x 4 bytes in registers, and feeds
// column n0 + 4r + j to instruction j (j = 0..3); one block therefore covers
// 64 columns.  FAST: M % (16 MT) == 0, N % 64 == 0, K % 64 == 0, 16-byte
// aligned A and C, lda multiple of 16, 4-byte aligned B, ldb multiple of 4,
// ldc of 4.
#pragma once

#include "device_common.h"

namespace tdi8 {

template <int MT, int NT, int WK, bool FAST>
__global__ void __launch_bounds__(WK * 64) gemm_skinny_kernel(GemmArgs g) {
    constexpr int BM = 16 * MT;
    constexpr int BN = 16 * NT;
    constexpr int TILES = MT * NT;

    __shared__ i32x4 red[WK][TILES][64];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int r16 = lane & 15;
    const int grp = lane >> 4;
    const int m0 = blockIdx.y * BM;
    const int n0 = blockIdx.x * BN;

    i32x4 acc[MT][NT];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NT; ++j) acc[i][j] = i32x4{0, 0, 0, 0};

    const int nss = (g.K + 255) / 256;
    for (int s = wave; s < nss; s += WK) {
        const int kb = 256 * s + 64 * grp;
        i32x4 xb[NT][4], xa[MT][4];
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            const int col = n0 + 16 * j + r16;
            const int8_t *p = g.B + static_cast<int64_t>(col) * g.ldb + kb;
#pragma unroll
            for (int q = 0; q < 4; ++q)
                xb[j][q] = FAST ? load16(p + 16 * q)
                                : load16_masked(p + 16 * q, col < g.N ? clamp16(g.K - (kb + 16 * q)) : 0);
        }
#pragma unroll
        for (int i = 0; i < MT; ++i) {
            const int row = m0 + 16 * i + r16;
            const int8_t *p = g.A + static_cast<int64_t>(row) * g.lda + kb;
#pragma unroll
            for (int q = 0; q < 4; ++q)
                xa[i][q] = FAST ? load16(p + 16 * q)
                                : load16_masked(p + 16 * q, row < g.M ? clamp16(g.K - (kb + 16 * q)) : 0);
        }
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int i = 0; i < MT; ++i)
#pragma unroll
                for (int j = 0; j < NT; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(xb[j][q], xa[i][q], acc[i][j], 0, 0, 0);
    }

#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NT; ++j) red[wave][i * NT + j][lane] = acc[i][j];
    __syncthreads();

    // Sum the WK partials; lane l of tile (i, j) holds D[n][m] for
    // m = l % 16, n = 4 (l / 16) .. +3, i.e. C[m][n .. n+3].
    for (int t = tid; t < TILES * 64; t += WK * 64) {
        const int tile = t >> 6;
        const int l = t & 63;
        i32x4 sum = red[0][tile][l];
#pragma unroll
        for (int w = 1; w < WK; ++w) sum += red[w][tile][l];
        const int m = m0 + 16 * (tile / NT) + (l & 15);
        const int n = n0 + 16 * (tile % NT) + 4 * (l >> 4);
        store4<FAST>(g, m, n, sum);
    }
}

template <int MT, int WK, bool FAST>
__global__ void __launch_bounds__(WK * 64) gemm_skinny_rr_kernel(GemmArgs g) {
    constexpr int BM = 16 * MT;
    constexpr int BN = 64;

    __shared__ i32x4 red[WK][MT * 4][64];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int r16 = lane & 15;
    const int grp = lane >> 4;
    const int m0 = blockIdx.y * BM;
    const int n0 = blockIdx.x * BN;
    const int col = n0 + 4 * r16;
    const int ncol = clamp4(g.N - col);

    i32x4 acc[MT][4];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = i32x4{0, 0, 0, 0};

    const int nss = (g.K + 63) / 64;
    for (int s = wave; s < nss; s += WK) {
        const int kb = 64 * s + 16 * grp;
        uint32_t w[16];
#pragma unroll
        for (int t = 0; t < 16; ++t) {
            const int k = kb + t;
            const int8_t *p = g.B + static_cast<int64_t>(k) * g.ldb + col;
            w[t] = FAST ? *reinterpret_cast<const uint32_t *>(p) : load4_masked(p, k < g.K ? ncol : 0);
        }
        i32x4 xb[4];
#pragma unroll
        for (int qd = 0; qd < 4; ++qd) {
            uint32_t t4[4];
            transpose4x4(&w[4 * qd], t4);
#pragma unroll
            for (int j = 0; j < 4; ++j) xb[j][qd] = static_cast<int32_t>(t4[j]);
        }
#pragma unroll
        for (int i = 0; i < MT; ++i) {
            const int row = m0 + 16 * i + r16;
            const int8_t *p = g.A + static_cast<int64_t>(row) * g.lda + kb;
            const i32x4 xa = FAST ? load16(p) : load16_masked(p, row < g.M ? clamp16(g.K - kb) : 0);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(xb[j], xa, acc[i][j], 0, 0, 0);
        }
    }

#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) red[wave][i * 4 + j][lane] = acc[i][j];
    __syncthreads();

    // Instruction j's lane l, register e holds D[n'][m] with m = l % 16 and
    // n' = 4 (l / 16) + e, i.e. column n0 + 4 n' + j.  Thread (i, l, e)
    // gathers the four j for one n' and stores C[m][n0 + 4 n' .. +3].
    for (int t = tid; t < MT * 64 * 4; t += WK * 64) {
        const int i = t / 256;
        const int l = (t / 4) & 63;
        const int e = t & 3;
        i32x4 v;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            int32_t sum = 0;
#pragma unroll
            for (int w = 0; w < WK; ++w) sum += red[w][i * 4 + j][l][e];
            v[j] = sum;
        }
        const int m = m0 + 16 * i + (l & 15);
        const int n = n0 + 4 * (4 * (l >> 4) + e);
        store4<FAST>(g, m, n, v);
    }
}

}  // namespace tdi8
