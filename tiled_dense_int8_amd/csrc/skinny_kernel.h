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
// Block: rows [m0, m0 + 16*MT), columns [n0, n0 + 16*NT), all of K.  K is
// cut into 256-byte super-steps; wave w takes the batches of SS consecutive
// super-steps starting at w*SS, w*SS + WK*SS, ...  A batch is loaded in one
// go (all of its B and A bytes requested before any is used, so a wave keeps
// SS*(NT+MT) KiB in flight and the whole B stream is requested almost at
// once), then consumed by four v_mfma_i32_16x16x64_i8 per super-step and
// instruction tile: instruction q of super-step s covers k = 256 s + 64 q
// .. +63, lane (r = lane % 16, g = lane / 16) holding k = 256 s + 64 q + 16 g
// .. +15 of its B column and of its A row (each load instruction reads 64
// contiguous bytes from each of 16 rows).
//
// gemm_skinny_kernel takes column-major B (K-contiguous columns).  FAST:
// N % (16 NT) == 0, K % 256 == 0, 16-byte aligned A, B, C, lda and ldb
// multiples of 16, ldc of 4.
//
// gemm_skinny_rr_kernel takes row-major B (N contiguous) in the predicated
// form.  There lane (r, g) reads, for the 16 rows k = 64*s + 16*g .. +15,
// the dword holding columns n0 + 4r .. +3, transposes the 16 x 4 bytes in
// registers, and feeds column n0 + 4r + j to instruction j (j = 0..3); one
// block therefore covers 64 columns.  Aligned row-major shapes go to the
// column-group form (the split form of the pipelined kernel, see
// kernel_table.h) when N and K divide into its groups and slices, else to
// gemm_skinny_rrlds_kernel below.
#pragma once

#include "device_common.h"
#include "rc_pipelined_kernel.h"  // LDS-DMA helpers

namespace tdi8 {

template <int MT, int NT, int WK, int SS, bool FAST>
__global__ void __launch_bounds__(WK * 64) gemm_skinny_kernel(GemmArgs g) {
    constexpr int BM = 16 * MT;
    constexpr int BN = 16 * NT;
    constexpr int TILES = MT * NT;

    __shared__ i32x4 red[WK][TILES][64];
    BlockStamp stamp;
    stamp.begin();

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int r16 = lane & 15;
    const int grp = lane >> 4;
    const int m0 = blockIdx.y * BM;
    const int n0 = blockIdx.x * BN;

    const int8_t *bp[NT];
    const int8_t *ap[MT];
    int bcol_ok[NT], arow_ok[MT];
#pragma unroll
    for (int j = 0; j < NT; ++j) {
        const int col = n0 + 16 * j + r16;
        bcol_ok[j] = FAST || col < g.N;
        bp[j] = g.B + static_cast<int64_t>(bcol_ok[j] ? col : 0) * g.ldb + 16 * grp;
    }
#pragma unroll
    for (int i = 0; i < MT; ++i) {
        const int row = m0 + 16 * i + r16;
        arow_ok[i] = FAST || row < g.M;
        ap[i] = g.A + static_cast<int64_t>(arow_ok[i] ? row : 0) * g.lda + 16 * grp;
    }

    i32x4 acc[MT][NT];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NT; ++j) acc[i][j] = i32x4{0, 0, 0, 0};

    const int nss = (g.K + 255) / 256;
    for (int s0 = wave * SS; s0 < nss; s0 += WK * SS) {
        i32x4 xb[SS][NT][4], xa[SS][MT][4];
#pragma unroll
        for (int u = 0; u < SS; ++u) {
            const int s = s0 + u;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int k = 256 * s + 64 * q + 16 * grp;  // this lane's first K
#pragma unroll
                for (int j = 0; j < NT; ++j) {
                    const int8_t *p = bp[j] + 256 * s + 64 * q;
                    if (FAST)
                        xb[u][j][q] = s < nss ? load16(p) : i32x4{0, 0, 0, 0};
                    else
                        xb[u][j][q] = load16_masked(p, (bcol_ok[j] && s < nss) ? clamp16(g.K - k) : 0);
                }
#pragma unroll
                for (int i = 0; i < MT; ++i) {
                    const int8_t *p = ap[i] + 256 * s + 64 * q;
                    if (FAST)
                        xa[u][i][q] = s < nss ? load16(p) : i32x4{0, 0, 0, 0};
                    else
                        xa[u][i][q] = load16_masked(p, (arow_ok[i] && s < nss) ? clamp16(g.K - k) : 0);
                }
            }
        }
        // every load of the batch is in flight before the first use
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < SS; ++u)
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int i = 0; i < MT; ++i)
#pragma unroll
                    for (int j = 0; j < NT; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(xb[u][j][q], xa[u][i][q], acc[i][j], 0, 0, 0);
    }
    stamp.loop_done();

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
    stamp.end(g);
}

// Unpredicated skinny kernel for column-major B (K a multiple of 16, A, B
// and C aligned).  The direct operand loads above read 16 rows x 64 bytes
// per instruction, which streams poorly from HBM; here every load
// instruction moves one whole kilobyte of one row of A or B straight into
// LDS (global_load_lds_dwordx4), so the stream is fully contiguous.  K is
// taken in chunks of KC bytes, two chunks in flight; a chunk's rows sit in
// LDS with a 32-byte pad (row stride KC + 32), so the 16 lanes that read
// one K position of 16 rows hit 16 different bank groups.  After a chunk
// lands, wave w consumes K positions w*KC/WK .. (w+1)*KC/WK - 1 of it with
// v_mfma_i32_16x16x64_i8 fed by ds_read_b128, and the WK partial sums are
// reduced in LDS at the end.  When A and B tiles have as many rows and all
// of K fits the two buffers, a second form below takes the loads with half
// the waves per operand and a single wait.
template <int MT, int NT, int WK, int KC>
__global__ void __launch_bounds__(WK * 64) gemm_skinny_lds_kernel(GemmArgs g) {
    constexpr int BM = 16 * MT;
    constexpr int BN = 16 * NT;
    constexpr int TILES = MT * NT;
    constexpr int ROWS = BM + BN;
    // LDS row stride: 32 bytes of padding (with 16 every operand read counted
    // four bank-conflict cycles; +32 measured 2% faster at 16 x 4096 x 4096,
    // +64 no better, +128 6% slower)
    constexpr int RS = KC + 32;
    constexpr int PIECES = KC / 1024;               // 1 KiB pieces per row and chunk
    constexpr int LOADS = ROWS * PIECES;            // wave instructions per chunk
    constexpr int LPW = LOADS / WK;
    constexpr int KW = KC / WK;                     // K positions per wave and chunk
    static_assert(KC % 1024 == 0 && LOADS % WK == 0 && KW % 64 == 0, "chunk must split evenly");
    static_assert(2 * ROWS * RS <= 160 * 1024 - TILES * 1024, "LDS budget");

#if defined(__HIP_DEVICE_COMPILE__)
    __shared__ __attribute__((aligned(1024))) int8_t buf[2][ROWS * RS];
    // Block sum, accumulated with LDS atomics; element e of lane l at
    // [tile][e][l], so the 64 lanes of one atomic hit 64 different banks.
    __shared__ int32_t red[TILES][4][64];
    BlockStamp stamp;
    stamp.begin();

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int r16 = lane & 15;
    const int grp = lane >> 4;
    const int m0 = blockIdx.y * BM;
    const int n0 = blockIdx.x * BN;
    const int nch = (g.K + KC - 1) / KC;
    // One block row: every B byte is read by one block only, A by all of
    // them; B then streams past the cache (4% at 16 x 8192 x 8192, neutral
    // at 16 x 4096 x 4096; with two block rows the hint cost 10%).  Taken
    // from the arguments, not gridDim: reading the grid size adds the
    // hidden argument block to the launch (72 -> 328 bytes, ~1% here).
    const bool b_once = g.tiles_m == 1;

    i32x4 acc[MT][NT];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NT; ++j) acc[i][j] = i32x4{0, 0, 0, 0};
    for (int t = tid; t < TILES * 64 * 4; t += WK * 64) (&red[0][0][0])[t] = 0;

    // Matrix work on the S chunks held in the two buffers from chunk c0 by
    // W waves, wave w taking K positions [w S KC / W, (w + 1) S KC / W) of
    // them (within one chunk: W is even).
    auto consume = [&](int c0, auto s_tag, auto w_tag) {
        constexpr int KWS = decltype(s_tag)::value * KC / decltype(w_tag)::value;
        static_assert(KWS % 64 == 0 && (KC % KWS == 0), "a wave's K range lies in one chunk");
        const int kw0 = wave * KWS;
        const int8_t *b = buf[(c0 + kw0 / KC) & 1];
#pragma unroll
        for (int kk = 0; kk < KWS; kk += 64) {
            const int k = kw0 % KC + kk + 16 * grp;
            i32x4 xa[MT], xb[NT];
#pragma unroll
            for (int i = 0; i < MT; ++i) xa[i] = *reinterpret_cast<const i32x4 *>(b + (16 * i + r16) * RS + k);
#pragma unroll
            for (int j = 0; j < NT; ++j) xb[j] = *reinterpret_cast<const i32x4 *>(b + (BM + 16 * j + r16) * RS + k);
#pragma unroll
            for (int i = 0; i < MT; ++i)
#pragma unroll
                for (int j = 0; j < NT; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(xb[j], xa[i], acc[i][j], 0, 0, 0);
        }
    };
    using One = std::integral_constant<int, 1>;
    using Two = std::integral_constant<int, 2>;

    // As many A rows as B rows and all of K within the two buffers (the
    // M = 16 headline, K <= 2 KC): waves [0, WK/2) move B and waves [WK/2,
    // WK) move A, so A (an L2 hit for all but the first blocks) never
    // waits behind B's HBM latency in the same wave (a wave's loads
    // complete in issue order); each operand's rows are requested row by
    // row, the pieces of a row in K order across both chunks (its requests
    // reach memory in address order); one wait, then the matrix work.
    // 16 x 4096 x 4096, column-major B: 5.7 -> 5.25 us against the general
    // loop below, measured side by side on one device.  Elsewhere the
    // general loop stays faster (longer K: 32 x 4096 x 8192 took 16.4 us
    // in this form against 11.8).
    constexpr bool SPLITW = BM == BN && WK % 2 == 0;
    // at most 8 waves take part (4 per operand: 16 x 4096 x 4096 ran 5.25 us
    // with 8 and 5.5 with 16); the others only keep the block's barriers
    constexpr int FW = WK < 8 ? WK : 8;
    if (SPLITW && nch <= 2) {
        constexpr int NW = FW / 2;                       // waves per operand
        constexpr int PR = 2 * PIECES;                   // pieces per row over both chunks
        const bool b_wave = wave < NW;
        const int rw = b_wave ? wave : wave - NW;
        const int8_t *base = b_wave ? g.B + static_cast<int64_t>(n0) * g.ldb : g.A + static_cast<int64_t>(m0) * g.lda;
        const int64_t ld = b_wave ? g.ldb : g.lda;
        const int valid = b_wave ? BN : g.M - m0;        // A rows past M read the zero chunk
        const int row0 = b_wave ? BM : 0;
        const int kdim = g.K;
        // rows of this wave's operand, pieces x = rw, rw + NW, ... of the
        // row-major enumeration; the 16-byte pieces at or past K of a last,
        // partial chunk (K a multiple of 16) read the zero chunk
        auto issue_rows = [&](auto nt_tag) {
            constexpr int NTF = decltype(nt_tag)::value;
            for (int x = rw; x < BM * PR; x += NW) {
                const int r = x / PR, pc = x % PR;
                const int k = pc * 1024 + 16 * lane;
                const int8_t *src = k < kdim && r < valid ? base + r * ld + k : zero_chunk;
                __builtin_amdgcn_global_load_lds(src, (lds_void_t *)(buf[pc / PIECES] + (row0 + r) * RS + (pc % PIECES) * 1024),
                                                 16, 0, NTF);
            }
        };
        if (wave < FW) {
            if (!b_wave)
                issue_rows(std::integral_constant<int, 0>{});
            else if (b_once)
                issue_rows(std::integral_constant<int, kLoadStream>{});
            else
                issue_rows(std::integral_constant<int, 0>{});
        }
        TDI8_WAIT_VMCNT(0);
        __syncthreads();
        if (wave < FW) {
            if (nch == 2)
                consume(0, Two{}, std::integral_constant<int, FW>{});
            else if (nch == 1)
                consume(0, One{}, std::integral_constant<int, FW>{});
        }
    } else {
        // A rows past M (a ragged M, e.g. M < 16) read the zero chunk (ok
        // false), and so do the 16-byte pieces at or past K of a last,
        // partial chunk (K a multiple of 16; kin: the piece's K offset
        // within a chunk).  Two chunks in flight.
        const int8_t *src[LPW];
        int dst_off[LPW], kin[LPW];
        bool ok[LPW];
#pragma unroll
        for (int i = 0; i < LPW; ++i) {
            const int x = i * WK + wave;
            const int row = x / PIECES;
            const int piece = x % PIECES;
            kin[i] = piece * 1024 + 16 * lane;
            ok[i] = row >= BM || m0 + row < g.M;
            src[i] = (row < BM ? g.A + static_cast<int64_t>(ok[i] ? m0 + row : m0) * g.lda
                               : g.B + static_cast<int64_t>(n0 + row - BM) * g.ldb) + piece * 1024 + 16 * lane;
            dst_off[i] = row * RS + piece * 1024;
        }
        auto issue = [&](int c) {
#pragma unroll
            for (int i = 0; i < LPW; ++i) {
                const int8_t *p = ok[i] && c * KC + kin[i] < g.K ? src[i] + c * KC : zero_chunk;
                if (b_once && (i * WK + wave) / PIECES >= BM)
                    __builtin_amdgcn_global_load_lds(p, (lds_void_t *)(buf[c & 1] + dst_off[i]), 16, 0, kLoadStream);
                else
                    __builtin_amdgcn_global_load_lds(p, (lds_void_t *)(buf[c & 1] + dst_off[i]), 16, 0, 0);
            }
        };
        if (nch > 0) issue(0);
        if (nch > 1) issue(1);
        for (int c = 0; c < nch; ++c) {
            if (c + 1 < nch) {
                TDI8_WAIT_VMCNT(LPW);
            } else {
                TDI8_WAIT_VMCNT(0);
            }
            block_barrier();
            const int8_t *b = buf[c & 1];
#pragma unroll
            for (int kk = 0; kk < KW; kk += 64) {
                const int k = wave * KW + kk + 16 * grp;
                i32x4 xa[MT], xb[NT];
#pragma unroll
                for (int i = 0; i < MT; ++i) xa[i] = *reinterpret_cast<const i32x4 *>(b + (16 * i + r16) * RS + k);
#pragma unroll
                for (int j = 0; j < NT; ++j)
                    xb[j] = *reinterpret_cast<const i32x4 *>(b + (BM + 16 * j + r16) * RS + k);
#pragma unroll
                for (int i = 0; i < MT; ++i)
#pragma unroll
                    for (int j = 0; j < NT; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(xb[j], xa[i], acc[i][j], 0, 0, 0);
            }
            if (c + 2 < nch) {
                TDI8_WAIT_LGKM0();
                block_barrier();  // every wave is done with this buffer
                issue(c + 2);
            }
        }
    }
    stamp.loop_done();

    // Sum the waves' partial tiles: integer addition is exact in any order,
    // so every wave adds its tile into one LDS copy with atomics.
    __syncthreads();
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NT; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) atomicAdd(&red[i * NT + j][e][lane], acc[i][j][e]);
    __syncthreads();
    for (int t = tid; t < TILES * 64; t += WK * 64) {
        const int tile = t >> 6;
        const int l = t & 63;
        const i32x4 sum = {red[tile][0][l], red[tile][1][l], red[tile][2][l], red[tile][3][l]};
        const int m = m0 + 16 * (tile / NT) + (l & 15);
        const int n = n0 + 16 * (tile % NT) + 4 * (l >> 4);
        if (m < g.M) store4<true>(g, m, n, sum);
    }
    stamp.end(g);
#endif
}

// Unpredicated skinny kernel for row-major B (used when N % (16 NT) == 0,
// K % KC == 0 and everything is 16-byte aligned).  Each block covers 16 NT
// columns (so that N = 4096 still gives 256 blocks); a column block's B is
// then 16 bytes of every K row.  One load instruction moves 64 such pieces,
// one per lane, into a 1 KiB LDS group holding 64 K rows of one 16-column
// sub-block; A rows move as whole kilobytes as in gemm_skinny_lds_kernel.
// The K-major B operand of v_mfma_i32_16x16x64_i8 is then gathered with
// ds_read_b64_tr_b8: within each 16-lane group, lanes 2r and 2r+1 address
// the two 8-byte halves of row r of an 8 x 16-byte block and lane c
// receives column c (eight K values).  Lane group q needs K rows
// 16q .. 16q+15 of the 64-row step, so row k' of a group is stored in slot
// (k' % 8) + 8 ((k' / 16) % 4) + 32 ((k' / 8) % 2): the eight rows one
// transpose read of group q touches are then 128 contiguous bytes at 128 q
// (low half) or 512 + 128 q (high half), and the lanes of one LDS pass hit
// 64 different banks.  Column blocks are renumbered so that the 8 blocks
// sharing one 128-byte line of a B row run on the same XCD (blocks are dealt
// to the 8 XCDs round-robin) and meet in its L2.
template <int MT, int NT, int WK, int KC>
__global__ void __launch_bounds__(WK * 64) gemm_skinny_rrlds_kernel(GemmArgs g) {
    constexpr int BM = 16 * MT;
    constexpr int BN = 16 * NT;
    constexpr int TILES = MT * NT;
    constexpr int RS = KC + 16;                     // LDS row stride of A
    constexpr int PIECES = KC / 1024;               // 1 KiB pieces per A row and chunk
    constexpr int A_LOADS = BM * PIECES;
    constexpr int GROUPS = KC / 64;                 // 64-row groups per B sub-block and chunk
    constexpr int LOADS = A_LOADS + NT * GROUPS;    // wave instructions per chunk
    constexpr int LPW = LOADS / WK;
    constexpr int KW = KC / WK;                     // K positions per wave and chunk
    constexpr int A_REGION = BM * RS;
    constexpr int STAGE = A_REGION + NT * KC * 16;
    static_assert(KC % 1024 == 0 && LOADS % WK == 0 && KW % 64 == 0, "chunk must split evenly");
    static_assert(2 * STAGE <= 160 * 1024 - TILES * 1024, "LDS budget");

#if defined(__HIP_DEVICE_COMPILE__)
    __shared__ __attribute__((aligned(1024))) int8_t buf[2][STAGE];
    __shared__ int32_t red[TILES][4][64];   // as in gemm_skinny_lds_kernel
    BlockStamp stamp;
    stamp.begin();

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int r16 = lane & 15;
    const int grp = lane >> 4;
    const int nb = g.tiles_n;  // the grid's width (from the arguments: reading gridDim adds the hidden argument block)
    const int cb = (nb & 7) == 0 ? (blockIdx.x & 7) * (nb >> 3) + (blockIdx.x >> 3) : blockIdx.x;
    const int m0 = blockIdx.y * BM;
    const int n0 = cb * BN;
    const int nch = (g.K + KC - 1) / KC;  // a last, partial chunk reads zero pieces past K

    // K row of this lane's piece within a 64-row group (inverse of the slot map)
    const int krow = (lane & 7) + 8 * (lane >> 5) + 16 * ((lane >> 3) & 3);
    const int8_t *src[LPW];
    int dst_off[LPW], kin[LPW];  // kin: the slot's K offset within a chunk
    bool is_b[LPW], ok[LPW];
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
        const int x = i * WK + wave;
        ok[i] = true;
        if (x < A_LOADS) {
            const int row = x / PIECES;
            const int piece = x % PIECES;
            kin[i] = piece * 1024 + 16 * lane;
            ok[i] = m0 + row < g.M;   // A rows past M read the zero chunk
            src[i] = g.A + static_cast<int64_t>(ok[i] ? m0 + row : m0) * g.lda + piece * 1024 + 16 * lane;
            dst_off[i] = row * RS + piece * 1024;
            is_b[i] = false;
        } else {
            const int xb = x - A_LOADS;
            const int j = xb / GROUPS;
            const int grp64 = xb % GROUPS;
            kin[i] = 64 * grp64 + krow;
            src[i] = g.B + static_cast<int64_t>(64 * grp64 + krow) * g.ldb + n0 + 16 * j;
            dst_off[i] = A_REGION + j * KC * 16 + grp64 * 1024;
            is_b[i] = true;
        }
    }
    auto issue = [&](int c) {
#pragma unroll
        for (int i = 0; i < LPW; ++i) {
            const int64_t off = is_b[i] ? static_cast<int64_t>(c) * KC * g.ldb : static_cast<int64_t>(c) * KC;
            const bool in = ok[i] && c * KC + kin[i] < g.K;
            __builtin_amdgcn_global_load_lds(in ? src[i] + off : zero_chunk, (lds_void_t *)(buf[c & 1] + dst_off[i]),
                                             16, 0, 0);
        }
    };

    // transpose-read offsets (within a 64-row group) of this lane: row r16/2, half r16%2
    const int tr_lo = ((r16 >> 1) + 8 * grp) * 16 + 8 * (r16 & 1);
    const int tr_hi = tr_lo + 32 * 16;

    i32x4 acc[MT][NT];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NT; ++j) acc[i][j] = i32x4{0, 0, 0, 0};

    for (int t = tid; t < TILES * 64 * 4; t += WK * 64) (&red[0][0][0])[t] = 0;
    if (nch > 0) issue(0);
    if (nch > 1) issue(1);
    for (int c = 0; c < nch; ++c) {
        if (c + 1 < nch) {
            TDI8_WAIT_VMCNT(LPW);
        } else {
            TDI8_WAIT_VMCNT(0);
        }
        block_barrier();
        const int8_t *b = buf[c & 1];
#pragma unroll
        for (int kk = 0; kk < KW; kk += 64) {
            const int kb = wave * KW + kk;
            i32x4 xa[MT], xb[NT];
#pragma unroll
            for (int i = 0; i < MT; ++i)
                xa[i] = *reinterpret_cast<const i32x4 *>(b + (16 * i + r16) * RS + kb + 16 * grp);
#pragma unroll
            for (int j = 0; j < NT; ++j) {
                const int8_t *base = b + A_REGION + j * KC * 16 + (kb >> 6) * 1024;
                typedef int v2i_t __attribute__((ext_vector_type(2)));
                typedef __attribute__((address_space(3))) v2i_t lds_v2i_t;
                const v2i_t lo = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i_t *)(base + tr_lo));
                const v2i_t hi = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i_t *)(base + tr_hi));
                xb[j] = i32x4{lo[0], lo[1], hi[0], hi[1]};
            }
#pragma unroll
            for (int i = 0; i < MT; ++i)
#pragma unroll
                for (int j = 0; j < NT; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(xb[j], xa[i], acc[i][j], 0, 0, 0);
        }
        if (c + 2 < nch) {
            TDI8_WAIT_LGKM0();
            block_barrier();  // every wave is done with this buffer
            issue(c + 2);
        }
    }
    stamp.loop_done();

    __syncthreads();
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NT; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) atomicAdd(&red[i * NT + j][e][lane], acc[i][j][e]);
    __syncthreads();
    for (int t = tid; t < TILES * 64; t += WK * 64) {
        const int tile = t >> 6;
        const int l = t & 63;
        const i32x4 sum = {red[tile][0][l], red[tile][1][l], red[tile][2][l], red[tile][3][l]};
        const int m = m0 + 16 * (tile / NT) + (l & 15);
        const int n = n0 + 16 * (tile % NT) + 4 * (l >> 4);
        if (m < g.M) store4<true>(g, m, n, sum);
    }
    stamp.end(g);
#endif
}

template <int MT, int WK, int SS, bool FAST>
__global__ void __launch_bounds__(WK * 64) gemm_skinny_rr_kernel(GemmArgs g) {
    constexpr int BM = 16 * MT;
    constexpr int BN = 64;

    __shared__ i32x4 red[WK][MT * 4][64];
    BlockStamp stamp;
    stamp.begin();

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

    // Batches of SS steps of 64 K: wave w takes steps w*SS .. w*SS+SS-1,
    // then (w + WK)*SS ..; all loads of a batch are issued before use.
    const int nss = (g.K + 63) / 64;
    for (int s0 = wave * SS; s0 < nss; s0 += WK * SS) {
        uint32_t w[SS][16];
        i32x4 xa[SS][MT];
#pragma unroll
        for (int u = 0; u < SS; ++u) {
            const int kb = 64 * (s0 + u) + 16 * grp;
#pragma unroll
            for (int t = 0; t < 16; ++t) {
                const int k = kb + t;
                const int8_t *p = g.B + static_cast<int64_t>(k < g.K ? k : 0) * g.ldb + col;
                if (FAST)
                    w[u][t] = k < g.K ? *reinterpret_cast<const uint32_t *>(p) : 0u;
                else
                    w[u][t] = load4_masked(p, k < g.K ? ncol : 0);
            }
#pragma unroll
            for (int i = 0; i < MT; ++i) {
                const int row = m0 + 16 * i + r16;
                const int8_t *p = g.A + static_cast<int64_t>(row < g.M ? row : 0) * g.lda + (kb < g.K ? kb : 0);
                xa[u][i] = FAST ? (kb < g.K ? load16(p) : i32x4{0, 0, 0, 0})
                                : load16_masked(p, row < g.M ? clamp16(g.K - kb) : 0);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < SS; ++u) {
            i32x4 xb[4];
#pragma unroll
            for (int qd = 0; qd < 4; ++qd) {
                uint32_t t4[4];
                transpose4x4(&w[u][4 * qd], t4);
#pragma unroll
                for (int j = 0; j < 4; ++j) xb[j][qd] = static_cast<int32_t>(t4[j]);
            }
#pragma unroll
            for (int i = 0; i < MT; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(xb[j], xa[u][i], acc[i][j], 0, 0, 0);
        }
    }
    stamp.loop_done();

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
    stamp.end(g);
}

}  // namespace tdi8
