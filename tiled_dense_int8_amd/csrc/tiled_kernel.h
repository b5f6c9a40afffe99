// General tiled int8 GEMM kernel for gfx950 (CDNA4), one instantiation per
// tile configuration.
//
// Block tile BM x BN of C, K walked in BK-deep tiles staged through LDS:
//  * tiling of global -> LDS -> registers cuts the re-reads of A and B by
//    the block and register tile sizes ("CUDA编程实践", section 3, the
//    global->shared and shared->register tiling paragraphs);
//  * two LDS stages: the next K tile is fetched into registers while the
//    current one is consumed, then written to the other stage, one barrier
//    per K tile (same section, the data-prefetch = double-buffer paragraph);
//  * 16-byte chunks of each LDS row are XOR-permuted by row so that the 16
//    lanes of a matrix-core operand read, which hit 16 consecutive rows at
//    one chunk column, touch 16 distinct 16-byte bank groups (the padding
//    idea of the contest write-up's "Padding 解决 bankconflict" section and
//    of the tutorial's section 1.3/1.4, done as a permutation so no LDS is
//    spent on padding);
//  * the contraction runs on the int8 matrix cores:
//    v_mfma_i32_32x32x32_i8 (MF = 32) or v_mfma_i32_16x16x64_i8 (MF = 16),
//    each wave owning MT x NT instruction tiles (register tiling; MT, NT are
//    the patent's m_tiles / n_tiles).
//
// Operand order.  The instruction computes D = X * Y with X's rows and Y's
// columns spread over lanes and the K values of an operand held 16 per lane.
// Both of our LDS tiles are K-contiguous (A as [BM][BK], B as [BN][BK]), so
// either can play X.  B plays X and A plays Y: D[n][m] = C[m][n], and the
// accumulator layout then gives each lane four consecutive n of one row m of
// C (16 bytes).  The epilogue stages C through LDS in row passes so that each
// store instruction writes whole rows (whole 128-byte lines, with the
// non-temporal hint).
//
// B layouts.  Column-major B (N x K, K contiguous) is staged like A.
// Row-major B (K x N, N contiguous) is staged as it lies, BK rows of BN bytes
// (16-byte chunks permuted by brow_swizzle), and its K-major operands are
// gathered with the transpose read ds_read_b64_tr_b8 (brow_frag_offsets).
//
// FAST = true: no predication; the dispatcher guarantees M % BM == 0,
// N % BN == 0, K % BK == 0, 16-byte aligned A, B, C and lda, ldb multiples
// of 16 (ldb of 4 for row-major B) and ldc of 4.  FAST = false: every load
// is bounded by M, N, K and any alignment is accepted; bytes past K read as
// zero, so the padded part of the last K tile adds exactly 0.
#pragma once

#include "device_common.h"

namespace tdi8 {

// Permutation of the 16-byte chunks of LDS row r (CPR chunks per row).
template <int CPR>
__device__ __forceinline__ int chunk_swizzle(int r) {
    static_assert(CPR == 4 || CPR == 8 || CPR == 16 || CPR == 32, "BK must be 64, 128, 256 or 512");
    if constexpr (CPR >= 16) return r & 15;
    if constexpr (CPR == 8) return (r & 7) ^ ((r >> 3) & 1);
    else return ((r >> 1) & 3) ^ ((r >> 3) & 1);
}

// Permutation of the 16-byte chunks of a row-major B row k in LDS (BN bytes
// per row): even values only, varying with k so that the eight rows read by
// one 16-lane group of a transpose read land on distinct bank groups.
template <int BN>
__device__ __forceinline__ int brow_swizzle(int k) {
    constexpr int CPRB = BN / 16;
    constexpr int P = BN >= 256 ? 1 : 256 / BN;  // rows sharing one 256-byte bank window
    return 2 * ((k / P) % (CPRB / 2));
}

// Row-major B tile [BK][BN] in LDS (chunks permuted by brow_swizzle): byte
// offsets, within the B region and for K step 0, of the two transpose reads
// (ds_read_b64_tr_b8) that gather lane `lane`'s K-major operand for the
// instruction tile whose columns start at ncol.  In each 16-lane group,
// lanes 2r and 2r+1 address the two 8-byte halves of row r of an 8 x 16-byte
// block and lane c receives column c (eight K values).  For the 32x32x32
// operand, lane l (group q = l / 16, c = l % 16) needs column ncol + l % 32
// and K = 16 (l / 32) .. +15: group q reads columns 16 (q % 2) .. +15 of K
// rows 16 (q / 2) + (0..7) and then + 8.  For the 16x16x64 operand lane l
// needs column ncol + l % 16 and K = 16 q .. +15.  K step ks lies
// ks * KSTEP * BN bytes further on; the swizzle's period (8 rows, 16 for
// BN = 512) divides KSTEP.
template <int MF, int BN>
__device__ __forceinline__ void brow_frag_offsets(int lane, int ncol, int &lo, int &hi) {
    const int q = lane >> 4, c = lane & 15;
    const int colgrp = MF == 32 ? (q & 1) : 0;
    const int kgrp = MF == 32 ? (q >> 1) : q;
    const int nb = ncol + 16 * colgrp;
    const int k0 = 16 * kgrp + (c >> 1);
    const int k1 = k0 + 8;
    lo = k0 * BN + 16 * ((nb >> 4) ^ brow_swizzle<BN>(k0)) + 8 * (c & 1);
    hi = k1 * BN + 16 * ((nb >> 4) ^ brow_swizzle<BN>(k1)) + 8 * (c & 1);
}

// The two halves of a transposed operand fragment, read at p0 and p1 (LDS).
__device__ __forceinline__ i32x4 read_tr_frag(const int8_t *p0, const int8_t *p1) {
    typedef int v2i_t __attribute__((ext_vector_type(2)));
    typedef __attribute__((address_space(3))) v2i_t lds_v2i_t;
    const v2i_t lo = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i_t *)(p0));
    const v2i_t hi = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i_t *)(p1));
    return i32x4{lo[0], lo[1], hi[0], hi[1]};
}

template <int MF>
struct Mfma;

template <>
struct Mfma<32> {
    using Acc = i32x16;
    static constexpr int KSTEP = 32;  // K per instruction
    static __device__ __forceinline__ Acc run(i32x4 x, i32x4 y, Acc c) {
        return __builtin_amdgcn_mfma_i32_32x32x32_i8(x, y, c, 0, 0, 0);
    }
};

template <>
struct Mfma<16> {
    using Acc = i32x4;
    static constexpr int KSTEP = 64;
    static __device__ __forceinline__ Acc run(i32x4 x, i32x4 y, Acc c) {
        return __builtin_amdgcn_mfma_i32_16x16x64_i8(x, y, c, 0, 0, 0);
    }
};

// Sixteen consecutive reduction positions kk .. kk+15 of one implicit-GEMM
// convolution row, gathered byte by byte (any channel count, any alignment):
// position k is channel c of tap (r, s), k = (r S + s) C + c, read from the
// image at (ih0 + r dh, iw0 + s dw); outside the image or past R S C it is 0.
__device__ __forceinline__ i32x4 conv_gather16(const int8_t *img, int ih0, int iw0, int kk, const ConvParams &cv) {
    uint32_t w[4] = {0u, 0u, 0u, 0u};
    int rs = fast_div(kk, cv.c_div);
    int c = kk - rs * cv.C;
    int r = fast_div(rs, cv.s_div);
    int s = rs - r * cv.S;
#pragma unroll
    for (int t = 0; t < 16; ++t) {
        const int ih = ih0 + r * cv.dh;
        const int iw = iw0 + s * cv.dw;
        if (kk + t < cv.rsc && static_cast<unsigned>(ih) < static_cast<unsigned>(cv.H) &&
            static_cast<unsigned>(iw) < static_cast<unsigned>(cv.W)) {
            const uint32_t b = static_cast<uint8_t>(img[(static_cast<int64_t>(ih) * cv.W + iw) * cv.C + c]);
            w[t >> 2] |= b << (8 * (t & 3));
        }
        if (++c == cv.C) {
            c = 0;
            if (++s == cv.S) {
                s = 0;
                ++r;
            }
        }
    }
    return i32x4{static_cast<int>(w[0]), static_cast<int>(w[1]), static_cast<int>(w[2]), static_cast<int>(w[3])};
}

// Run form of the gather (dw = 1): filter row r's run of S C bytes (taps
// s = 0 .. S-1, channels c) is padded to runp 16-byte pieces, so the
// reduction is R runp pieces and position kk is byte 16 j + kk % 16 of run r,
// with kk / 16 = r runp + j.  For one output pixel a run lies contiguously in
// image row ih0 + r dh from column iw0, so a piece is one masked load of its
// bytes that belong to taps inside the image (the dword reads of
// load16_masked stay on the pages of the wanted bytes) moved up to its place;
// taps outside the image, rows outside it and the padding are 0.
__device__ __forceinline__ i32x4 conv_run16(const int8_t *img, int ih0, int iw0, int kk, const ConvParams &cv) {
    const int pi = kk >> 4;
    const int r = fast_div(pi, cv.runp_div);
    const int j16 = 16 * (pi - r * cv.runp);
    const int ih = ih0 + r * cv.dh;
    if (r >= cv.R || static_cast<unsigned>(ih) >= static_cast<unsigned>(cv.H)) return i32x4{0, 0, 0, 0};
    const int s_lo = iw0 < 0 ? -iw0 : 0;                  // first tap inside the image
    const int s_hi = cv.W - iw0 < cv.S ? cv.W - iw0 : cv.S;  // one past the last
    const int lo = j16 > s_lo * cv.C ? j16 : s_lo * cv.C;
    int hi = j16 + 16 < cv.run ? j16 + 16 : cv.run;
    hi = hi < s_hi * cv.C ? hi : s_hi * cv.C;
    if (hi <= lo) return i32x4{0, 0, 0, 0};
    const int8_t *p = img + (static_cast<int64_t>(ih) * cv.W + iw0) * cv.C + lo;
    return shift_up_bytes(load16_masked(p, hi - lo), lo - j16);
}

// SRC 0: the product of the operands described by g.  SRC 1: implicit-GEMM
// convolution (A rows gathered from the NHWC image by conv_gather16, B the
// KRSC filters as column-major K x R S C, C the N P Q x K output).
// Whether a tile can take the deep-prefetch loop: A and B tiles split into
// whole 16-byte loads per thread, at most four per thread and K tile (a
// larger set would not fit the register budget of the tile's occupancy).
constexpr bool deep_prefetch_fits(int bm, int bn, int bk, int threads) {
    return (bm * bk / 16) % threads == 0 && (bn * bk / 16) % threads == 0 &&
           (bm * bk / 16) / threads + (bn * bk / 16) / threads <= 4;
}

// DEEP: the K loop with two register sets of loads in flight (below); the
// dispatcher runs it for column-major B when the grid holds at most one
// block per compute unit, K >= 16 and there are at least three K tiles.
template <int MF, int WM, int WN, int MT, int NT, int BK, bool BCOL, bool FAST, int SRC, bool DEEP = false>
__device__ __forceinline__ void tiled_body(const GemmArgs &g, const ConvParams &cv) {
    static_assert(SRC == 0 || (BCOL && !FAST), "the gathered convolution is the predicated column-major form");
    constexpr int NTH = WM * WN * 64;
    constexpr int BM = WM * MF * MT;
    constexpr int BN = WN * MF * NT;
    constexpr int CPR = BK / 16;                  // 16-byte chunks per LDS row
    constexpr int A_BYTES = BM * BK;
    constexpr int STAGE = (BM + BN) * BK;
    constexpr int A_CHUNKS = BM * CPR;
    constexpr int B_CHUNKS = BN * CPR;
    constexpr int A_PER = (A_CHUNKS + NTH - 1) / NTH;
    constexpr int B_PER = (B_CHUNKS + NTH - 1) / NTH;
    constexpr int CPRB = BN / 16;                 // 16-byte chunks per row-major B row
    static_assert(BCOL || CPRB >= 4, "row-major B tile at least 64 columns wide");
    constexpr int KSTEPS = BK / Mfma<MF>::KSTEP;
    using Acc = typename Mfma<MF>::Acc;

    __shared__ __attribute__((aligned(16))) int8_t lds[2 * STAGE];
    BlockStamp stamp;
    stamp.begin();

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave / WN;
    const int wn = wave % WN;
    const int tm = blockIdx.x / g.tiles_n;
    const int tn = blockIdx.x % g.tiles_n;
    const int m0 = tm * BM;
    const int n0 = tn * BN;

    Acc acc[MT][NT];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NT; ++j) acc[i][j] = Acc{};

    i32x4 ra[A_PER];
    i32x4 rb[B_PER];

    // Convolution: image base and tap (0, 0) position of each A slot's row
    // (row past M: a null base, gathered as zeros).
    [[maybe_unused]] const int8_t *cimg[SRC == 1 ? A_PER : 1];
    [[maybe_unused]] int cih[SRC == 1 ? A_PER : 1], ciw[SRC == 1 ? A_PER : 1];
    if constexpr (SRC == 1) {
#pragma unroll
        for (int i = 0; i < A_PER; ++i) {
            const int row = m0 + (tid + i * NTH) / CPR;
            const int pq = cv.P * cv.Q;
            const int mm = row < g.M ? row : 0;
            const int img = mm / pq;
            const int p = (mm - img * pq) / cv.Q;
            const int q = mm - img * pq - p * cv.Q;
            cimg[i] = row < g.M ? g.A + static_cast<int64_t>(img) * cv.H * cv.W * cv.C : nullptr;
            cih[i] = p * cv.sh - cv.ph;
            ciw[i] = q * cv.sw - cv.pw;
        }
    }

    // Global -> registers for K tile starting at k0.
    auto fetch = [&](int k0) {
#pragma unroll
        for (int i = 0; i < A_PER; ++i) {
            const int q = tid + i * NTH;
            if (A_CHUNKS % NTH == 0 || q < A_CHUNKS) {
                const int r = q / CPR;
                const int c = (q % CPR) ^ chunk_swizzle<CPR>(r);
                const int row = m0 + r;
                const int kk = k0 + 16 * c;
                if constexpr (SRC == 1) {
                    ra[i] = !cimg[i] ? i32x4{0, 0, 0, 0}
                            : cv.run ? conv_run16(cimg[i], cih[i], ciw[i], kk, cv)
                                     : conv_gather16(cimg[i], cih[i], ciw[i], kk, cv);
                } else {
                    const int8_t *p = g.A + static_cast<int64_t>(row) * g.lda + kk;
                    ra[i] = FAST ? load16(p) : load16_masked(p, row < g.M ? clamp16(g.K - kk) : 0);
                }
            }
        }
        if constexpr (BCOL) {
#pragma unroll
            for (int i = 0; i < B_PER; ++i) {
                const int q = tid + i * NTH;
                if (B_CHUNKS % NTH == 0 || q < B_CHUNKS) {
                    const int r = q / CPR;
                    const int c = (q % CPR) ^ chunk_swizzle<CPR>(r);
                    const int col = n0 + r;
                    const int kk = k0 + 16 * c;
                    if (SRC == 1 && cv.run) {
                        // run form: piece j of filter row r of output channel col
                        const int pi = kk >> 4;
                        const int r = fast_div(pi, cv.runp_div);
                        const int j16 = 16 * (pi - r * cv.runp);
                        const int8_t *p = g.B + static_cast<int64_t>(col) * g.ldb + r * cv.run + j16;
                        const int nb = cv.run - j16 < 16 ? cv.run - j16 : 16;
                        rb[i] = load16_masked(p, col < g.N && kk < g.K ? nb : 0);
                    } else {
                        const int8_t *p = g.B + static_cast<int64_t>(col) * g.ldb + kk;
                        rb[i] = FAST ? load16(p) : load16_masked(p, col < g.N ? clamp16(g.K - kk) : 0);
                    }
                }
            }
        } else {
            // Row-major B: slot q of the tile holds row k = q / CPRB, source
            // chunk (q % CPRB) ^ brow_swizzle(k), i.e. 16 consecutive columns.
#pragma unroll
            for (int i = 0; i < B_PER; ++i) {
                const int q = tid + i * NTH;
                if (B_CHUNKS % NTH == 0 || q < B_CHUNKS) {
                    const int k = q / CPRB;
                    const int c = (q % CPRB) ^ brow_swizzle<BN>(k);
                    const int kk = k0 + k;
                    const int col = n0 + 16 * c;
                    const int8_t *p = g.B + static_cast<int64_t>(kk) * g.ldb + col;
                    rb[i] = FAST ? load16(p) : load16_masked(p, kk < g.K ? clamp16(g.N - col) : 0);
                }
            }
        }
    };

    // Registers -> LDS stage s.
    auto stash = [&](int s) {
        int8_t *base = lds + s * STAGE;
#pragma unroll
        for (int i = 0; i < A_PER; ++i) {
            const int q = tid + i * NTH;
            if (A_CHUNKS % NTH == 0 || q < A_CHUNKS)
                *reinterpret_cast<i32x4 *>(base + 16 * q) = ra[i];
        }
#pragma unroll
        for (int i = 0; i < B_PER; ++i) {
            const int q = tid + i * NTH;
            if (B_CHUNKS % NTH == 0 || q < B_CHUNKS)
                *reinterpret_cast<i32x4 *>(base + A_BYTES + 16 * q) = rb[i];
        }
    };

    // Row-major B: LDS offsets of this lane's transpose reads (K step 0).
    [[maybe_unused]] int offbt[BCOL ? 1 : NT][2];
    if constexpr (!BCOL) {
#pragma unroll
        for (int j = 0; j < NT; ++j) brow_frag_offsets<MF, BN>(lane, wn * (NT * MF) + j * MF, offbt[j][0], offbt[j][1]);
    }

    // Matrix-core work on LDS stage s.
    auto compute = [&](int s) {
        const int8_t *As = lds + s * STAGE;
        const int8_t *Bs = As + A_BYTES;
        const int lrow = lane % MF;
        const int lgrp = lane / MF;
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) {
            const int c = ks * (Mfma<MF>::KSTEP / 16) + lgrp;
            i32x4 xa[MT], xb[NT];
#pragma unroll
            for (int i = 0; i < MT; ++i) {
                const int r = wm * (MT * MF) + i * MF + lrow;
                xa[i] = *reinterpret_cast<const i32x4 *>(As + r * BK + 16 * (c ^ chunk_swizzle<CPR>(r)));
            }
#pragma unroll
            for (int j = 0; j < NT; ++j) {
                if constexpr (BCOL) {
                    const int r = wn * (NT * MF) + j * MF + lrow;
                    xb[j] = *reinterpret_cast<const i32x4 *>(Bs + r * BK + 16 * (c ^ chunk_swizzle<CPR>(r)));
                } else {
                    constexpr int KSTEP = Mfma<MF>::KSTEP;
                    xb[j] = read_tr_frag(Bs + offbt[j][0] + ks * KSTEP * BN, Bs + offbt[j][1] + ks * KSTEP * BN);
                }
            }
#pragma unroll
            for (int i = 0; i < MT; ++i)
#pragma unroll
                for (int j = 0; j < NT; ++j) acc[i][j] = Mfma<MF>::run(xb[j], xa[i], acc[i][j]);
        }
    };

    const int nk = (g.K + BK - 1) / BK;
    if constexpr (DEEP) {
        static_assert(SRC == 0 && !FAST && BCOL && deep_prefetch_fits(BM, BN, BK, NTH),
                      "deep prefetch: column-major B, whole load sets of at most four loads per thread");
        // Deep prefetch (K >= 16, column-major B): PD register sets hold the
        // K tiles in flight, so a tile's loads are issued PD iterations
        // before it is stashed instead of one (PD = 2: of 2, 3 and 4 sets,
        // two were fastest on 512 x 512 x 4097, 2000 x 2000 x 2001 and
        // 1000 x 3000 x 777, where two blocks per compute unit already
        // load at the rate of its misaligned 16-byte loads).  Every set is filled by the
        // same unconditional 16-byte loads, whatever the tile (a fixed load
        // count per set keeps the compiler's waits counting only the set
        // being stashed), from addresses that are always inside the
        // operands:
        //  * rows past M or N read row M-1 or N-1: they only reach C rows or
        //    columns past M or N, which are never stored;
        //  * in the last K tile, when K is not a multiple of BK, a chunk
        //    that ends past K is read from the row's last 16 bytes,
        //    [K-16, K), and moved down to its place at the stash, the bytes
        //    past K becoming zero (shift_down_bytes); a chunk wholly past K
        //    reads the row's first 16 bytes and becomes zero.
        // The barrier between K tiles waits on LDS only (block_barrier):
        // __syncthreads() would also wait for the loads still in flight.
        constexpr int PD = 2;
        // the dispatcher guarantees both (a launch without them would
        // leave C as it was)
        if (g.K >= 16 && nk >= PD + 1) {
            const int nfull = g.K / BK;  // K tiles wholly inside K; tile nfull (if any) is the tail
            const int8_t *arow[A_PER];
            const int8_t *brow[B_PER];
            int acol[A_PER], bcol[B_PER];
#pragma unroll
            for (int i = 0; i < A_PER; ++i) {
                const int q = tid + i * NTH;
                const int r = q / CPR;
                acol[i] = 16 * ((q % CPR) ^ chunk_swizzle<CPR>(r));
                const int row = m0 + r < g.M ? m0 + r : g.M - 1;
                arow[i] = g.A + static_cast<int64_t>(row) * g.lda;
            }
#pragma unroll
            for (int i = 0; i < B_PER; ++i) {
                const int q = tid + i * NTH;
                const int r = q / CPR;
                bcol[i] = 16 * ((q % CPR) ^ chunk_swizzle<CPR>(r));
                const int col = n0 + r < g.N ? n0 + r : g.N - 1;
                brow[i] = g.B + static_cast<int64_t>(col) * g.ldb;
            }
            i32x4 qa[PD][A_PER], qb[PD][B_PER];
            int tsa[A_PER] = {}, tsb[B_PER] = {};  // tail tile: bytes to move each chunk down (16: zero)
            // Row offset of the chunk at kk: in place, except in the tail
            // tile, where a chunk ending past K reads [K-16, K) and one
            // wholly past K reads [0, 16), then moves down by 16 - nv bytes
            // (nv valid bytes stay, the rest becomes zero).  Tiles j >= nk
            // (the loop runs whole groups of PD iterations) read the
            // operands' first 16 bytes: the same loads, one cache line per
            // instruction, never stashed.  The choices are selects on
            // uniform values, with the loads after them: branches around
            // the address arithmetic let the compiler move the loads into
            // the branches, and its waits then count none of them.
            auto pick = [&](const int8_t *row, const int8_t *dummy, int kk, bool tail, bool live, int &shift) {
                const int nv = clamp16(g.K - kk);
                const int toff = nv == 16 ? kk : (nv > 0 ? g.K - 16 : 0);
                shift = tail ? 16 - nv : shift;
                const int8_t *p = row + (tail ? toff : kk);
                return live ? p : dummy;
            };
            auto fetch_deep = [&](int j, i32x4 (&xa)[A_PER], i32x4 (&xb)[B_PER]) {
                const int k0 = j * BK;
                const bool tail = j == nfull;
                const bool live = j < nk;
                const int8_t *pa[A_PER];
                const int8_t *pb[B_PER];
#pragma unroll
                for (int i = 0; i < A_PER; ++i) pa[i] = pick(arow[i], g.A, k0 + acol[i], tail, live, tsa[i]);
#pragma unroll
                for (int i = 0; i < B_PER; ++i) pb[i] = pick(brow[i], g.B, k0 + bcol[i], tail, live, tsb[i]);
#pragma unroll
                for (int i = 0; i < A_PER; ++i) xa[i] = load16_unaligned(pa[i]);
#pragma unroll
                for (int i = 0; i < B_PER; ++i) xb[i] = load16_unaligned(pb[i]);
            };
            auto stash_deep = [&](int j, const i32x4 (&xa)[A_PER], const i32x4 (&xb)[B_PER]) {
                int8_t *base = lds + (j & 1) * STAGE;
                if (j == nfull) {
#pragma unroll
                    for (int i = 0; i < A_PER; ++i)
                        *reinterpret_cast<i32x4 *>(base + 16 * (tid + i * NTH)) = shift_down_bytes(xa[i], tsa[i]);
#pragma unroll
                    for (int i = 0; i < B_PER; ++i)
                        *reinterpret_cast<i32x4 *>(base + A_BYTES + 16 * (tid + i * NTH)) =
                            shift_down_bytes(xb[i], tsb[i]);
                } else {
#pragma unroll
                    for (int i = 0; i < A_PER; ++i) *reinterpret_cast<i32x4 *>(base + 16 * (tid + i * NTH)) = xa[i];
#pragma unroll
                    for (int i = 0; i < B_PER; ++i)
                        *reinterpret_cast<i32x4 *>(base + A_BYTES + 16 * (tid + i * NTH)) = xb[i];
                }
            };
            // Tile j lives in set j % PD.  Prologue: tiles 0 .. PD-1 in
            // flight, tile 0 stashed and its set refilled with tile PD.
            static_for<PD>([&](auto uc) {
                constexpr int u = decltype(uc)::value;
                fetch_deep(u, qa[u], qb[u]);
            });
            stash_deep(0, qa[0], qb[0]);
            fetch_deep(PD, qa[0], qb[0]);
            TDI8_WAIT_LGKM0();
            block_barrier();
            // Iteration t: tile t's matrix work, tile t+1 to the other LDS
            // stage, its set refilled with tile t+1+PD, one barrier on LDS
            // only.  Whole groups of PD iterations, so that set indices are
            // compile-time and every iteration issues the same loads; the
            // iterations past the last tile only load (uniform branches
            // around LDS and matrix work leave the load sequence fixed).
            const int groups = (nk + PD - 1) / PD;
            for (int t0 = 0; t0 < groups * PD; t0 += PD) {
                static_for<PD>([&](auto uc) {
                    constexpr int U = (decltype(uc)::value + 1) % PD;
                    const int t = t0 + decltype(uc)::value;
                    if (t < nk) compute(t & 1);
                    if (t + 1 < nk) stash_deep(t + 1, qa[U], qb[U]);
                    fetch_deep(t + 1 + PD, qa[U], qb[U]);
                    TDI8_WAIT_LGKM0();
                    block_barrier();
                });
            }
        }
    }
    if (!DEEP && nk > 0) {
        fetch(0);
        stash(0);
        __syncthreads();
        for (int t = 0; t < nk; ++t) {
            if (t + 1 < nk) fetch((t + 1) * BK);
            compute(t & 1);
            if (t + 1 < nk) stash((t + 1) & 1);
            __syncthreads();
        }
    }
    stamp.loop_done();

    // Epilogue: lane holds D[n][m] = C[m][n] with four consecutive n per
    // group of four accumulator registers.  32x32 tiles go through the LDS
    // stages (free after the loop's last barrier) in passes of RP rows, so
    // each store instruction writes whole rows, with the non-temporal hint.
    if constexpr (MF == 32) {
        constexpr int RS = BN + 4;  // int32 per LDS row; the pad spreads the 32 rows of a write over the banks
        constexpr int RP0 = ((2 * STAGE) / (RS * 4)) / MF * MF;
        constexpr int RP = RP0 < BM ? RP0 : BM;
        static_assert(RP >= MF, "stage buffers hold at least one instruction tile of rows");
        int32_t *cl = reinterpret_cast<int32_t *>(lds);
        for (int p0 = 0; p0 < BM; p0 += RP) {
            __syncthreads();
#pragma unroll
            for (int i = 0; i < MT; ++i) {
                const int rb = wm * (MT * MF) + i * MF;
                if (rb < p0 || rb >= p0 + RP) continue;
#pragma unroll
                for (int j = 0; j < NT; ++j) {
                    const int cb = wn * (NT * MF) + j * MF;
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int r = rb - p0 + (lane & 31);
                        const int c = cb + 8 * q + 4 * (lane >> 5);
                        *reinterpret_cast<i32x4 *>(cl + r * RS + c) =
                            i32x4{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
                    }
                }
            }
            __syncthreads();
            const int rows = BM - p0 < RP ? BM - p0 : RP;
            for (int idx = tid; idx < rows * (BN / 4); idx += NTH) {
                const int r = idx / (BN / 4);
                const int c4 = idx - r * (BN / 4);
                store4_nt<FAST>(g, m0 + p0 + r, n0 + 4 * c4, *reinterpret_cast<const i32x4 *>(cl + r * RS + 4 * c4));
            }
        }
    } else {
#pragma unroll
        for (int i = 0; i < MT; ++i) {
#pragma unroll
            for (int j = 0; j < NT; ++j) {
                const int m = m0 + wm * (MT * MF) + i * MF + (lane & 15);
                const int n = n0 + wn * (NT * MF) + j * MF + 4 * (lane >> 4);
                store4<FAST>(g, m, n, acc[i][j]);
            }
        }
    }
    stamp.end(g);
}

template <int MF, int WM, int WN, int MT, int NT, int BK, bool BCOL, bool FAST>
__global__ void __launch_bounds__(WM * WN * 64) gemm_tiled_kernel(GemmArgs g) {
    tiled_body<MF, WM, WN, MT, NT, BK, BCOL, FAST, 0>(g, ConvParams{});
}

// The predicated column-major-B kernel with the deep-prefetch K loop.
template <int MF, int WM, int WN, int MT, int NT, int BK>
__global__ void __launch_bounds__(WM * WN * 64) gemm_tiled_prefetch_kernel(GemmArgs g) {
    tiled_body<MF, WM, WN, MT, NT, BK, true, false, 0, true>(g, ConvParams{});
}

// Implicit-GEMM convolution for any channel count and alignment: the
// predicated kernel with A gathered into registers, in 16-byte pieces of
// filter-row runs (conv_run16, dw = 1) or byte by byte (conv_gather16); the
// DMA form needs 16-byte chunks of 16 channels.
template <int MF, int WM, int WN, int MT, int NT, int BK>
__global__ void __launch_bounds__(WM * WN * 64) conv_gather_kernel(GemmArgs g, ConvParams cv) {
    tiled_body<MF, WM, WN, MT, NT, BK, true, false, 1>(g, cv);
}

}  // namespace tdi8
