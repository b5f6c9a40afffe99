// Unpredicated int8 GEMM kernel on gfx950: the form the dispatcher uses when
// the operands and leading dimensions are 16-byte aligned and K (and, for
// row-major B, N) is a multiple of 16: chunks outside the operands read a
// zero chunk and the stores of a partial tile are masked.
// A (row-major) and column-major B are K-contiguous, so their tiles go from
// HBM to LDS as K-contiguous rows.  Row-major B (BROW) is copied as it lies,
// BK rows of BN contiguous bytes, and its operand fragments are gathered
// K-major out of LDS with the transpose read ds_read_b64_tr_b8, so neither
// layout is staged or transposed in registers.
//
// Differences from gemm_tiled_kernel:
//  * global -> LDS with global_load_lds_dwordx4: each wave instruction moves
//    1 KiB straight into LDS (lane l's 16 bytes land at l*16 of the block),
//    so no VGPRs hold staged tiles and no ds_write is issued;
//  * STAGES LDS buffers; one barrier per K tile both publishes the next
//    tile and frees the buffer just consumed, which is refilled at once with
//    the tile STAGES ahead (prefetch = double buffering generalised;
//    "CUDA编程实践" section 3, the data-prefetch paragraph);
//  * instruction operands are prefetched one group of K steps ahead in
//    registers (step_group: about four matrix instructions per group); the
//    first group of the next K tile is read right after the barrier, under
//    the last group's matrix-core work;
//  * C leaves through LDS in row passes, every store instruction writing
//    whole 128-byte lines with the non-temporal hint (store4_nt);
//  * blocks are ordered so that the blocks resident on one XCD (workgroups
//    are dealt to the 8 XCDs round-robin) cover a compact group of tiles
//    and share A and B rows in that XCD's L2 (the contest write-up's
//    "Swizzle 线程块映射" idea; its point that flat waves of blocks lose L2
//    reuse is the "矩阵维度高度不均衡" paragraph).
#pragma once

#include <type_traits>

#include "device_common.h"
#include "tiled_kernel.h"

namespace tdi8 {

typedef __attribute__((address_space(3))) void lds_void_t;

// Sixteen zero bytes in device memory: the DMA source of chunks that lie
// outside the operand (zero padding of the convolution, K and row tails).
static __device__ __attribute__((aligned(16))) const int8_t zero_chunk[16] = {};

// Tile coordinates of block `bid` in XCD-grouped order.
__device__ __forceinline__ void tile_of_block(const GemmArgs &g, int bid, int &tm, int &tn) {
    const int total = g.tiles_m * g.tiles_n;
    int l = bid;
    if ((total & 7) == 0) l = (bid & 7) * (total >> 3) + (bid >> 3);
    const int group_rows = 4;
    const int gsize = group_rows * g.tiles_n;
    const int first = (l / gsize) * group_rows;
    const int rows = min(g.tiles_m - first, group_rows);
    const int within = l % gsize;
    tm = first + within % rows;
    tn = within / rows;
}

// K steps handled as one group by the pipelined schedule: operand reads go out
// one group ahead and are waited for once per group, so a wave with few
// matrix instructions per K step (small tiles: f of them) still has about
// four in flight while its next reads land.  Groups per K tile stay even
// (the operand double buffer alternates by group).
constexpr int step_group(int ks, int f) {
    int g = 1;
    while (ks % (4 * g) == 0 && 2 * g * f <= 4) g *= 2;
    return g;
}

// SPLIT: the grid holds g.splits blocks per tile, slice s of a tile covering
// K range [s K / splits, (s + 1) K / splits) (with EDGE rounded to 16-byte
// chunks) and adding its partial sums into C (zeroed beforehand) with integer
// atomics: exact in any order.
// EDGE: M, N or K may end inside a tile (chunks outside the operands read the
// zero chunk, stores are masked); without it M, N and the K extent of a block
// are whole tiles and the kernel carries none of these tests.
// PERSIST: the grid holds nblocks blocks (at most one tile each at a time);
// block b computes tiles b, b + nblocks, b + 2 nblocks, ... of the same
// XCD-grouped order (with nblocks a multiple of 8 a block stays on one XCD
// and the blocks of an XCD keep walking one compact group of tiles).  Its
// K tiles form one stream across tiles: the LDS refill of the last K tiles
// of a tile already loads the next tile's first ones, and each finished
// tile leaves straight from the accumulation registers (no LDS pass, no
// barrier), so its stores drain while the matrix work of the next tile
// runs.  Whole tiles only (M, N and K multiples of the tile), GEMM source.
template <int MF, int WM, int WN, int MT, int NT, int BK, int STAGES, bool BROW, bool SPLIT, bool EDGE, int SRC,
          bool PERSIST = false>
__device__ __forceinline__ void pipelined_body(const GemmArgs &g, const ConvParams &cv, int nblocks = 1) {
    static_assert(SRC == 0 || (!BROW && !SPLIT), "the convolution source is column-major B, unsplit");
    static_assert(!PERSIST || (SRC == 0 && !SPLIT && !EDGE && MF == 32), "persistent form: whole tiles, GEMM");
    constexpr int NW = WM * WN;
    constexpr int BM = WM * MF * MT;
    constexpr int BN = WN * MF * NT;
    constexpr int CPR = BK / 16;
    constexpr int A_CHUNKS = BM * CPR;
    constexpr int STAGE = (BM + BN) * BK;
    constexpr int A_BYTES_ = BM * BK;
    constexpr int LOADS = STAGE / 1024;          // 1 KiB wave instructions per stage
    constexpr int LPW = LOADS / NW;              // per wave
    constexpr int KSTEP = Mfma<MF>::KSTEP;
    constexpr int KS = BK / KSTEP;
    constexpr int KC = KSTEP / 16;               // 16-byte chunks per lane group per step
    static_assert(LOADS % NW == 0, "stage must split evenly over the waves");
    static_assert(A_CHUNKS % 64 == 0, "A region must be whole wave instructions");
    static_assert(STAGES >= 2, "at least two stages");
    static_assert(KS % 2 == 0, "operand double buffer needs an even number of K steps per tile");
    constexpr int G = step_group(KS, MT * NT);   // K steps per operand group
    constexpr int KG = KS / G;                   // groups per K tile
    static_assert(KG % 2 == 0, "operand double buffer needs an even number of groups per tile");
    // A load slot reads A or B for every wave alike (the persistent form
    // shifts the two operands' pointers separately from tile to tile).
    static_assert(!PERSIST || (A_CHUNKS / 64) % NW == 0, "load slots split A and B by slot index");
    constexpr int CPRB = BN / 16;                // 16-byte chunks per row-major B row
    static_assert(!BROW || (CPRB >= 4 && (BK * BN) % 1024 == 0), "row-major B form");
    using Acc = typename Mfma<MF>::Acc;
#if defined(__HIP_DEVICE_COMPILE__)  // the host pass only needs the launch stub

    __shared__ __attribute__((aligned(1024))) int8_t lds[STAGES * STAGE];
    BlockStamp stamp;
    stamp.begin();

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int wm = wave / WN;
    const int wn = wave % WN;
    int bid = blockIdx.x;
    int kslice = g.K;    // K extent of this block
    int64_t k_begin = 0;
    if constexpr (SPLIT) {
        const int tiles = g.tiles_m * g.tiles_n;
        const int slice = bid / tiles;
        bid -= slice * tiles;
        if constexpr (EDGE) {
            // K a multiple of 16: slice s covers 16-byte chunks [s C / splits,
            // (s + 1) C / splits) of the C = K / 16, so slices differ by at
            // most one chunk (empty only when C < splits)
            const int64_t chunks = g.K / 16;
            k_begin = 16 * (slice * chunks / g.splits);
            kslice = static_cast<int>(16 * ((slice + 1) * chunks / g.splits) - k_begin);
        } else {
            kslice = g.K / g.splits;
            k_begin = static_cast<int64_t>(slice) * kslice;
        }
    }
    int tm, tn;
    tile_of_block(g, bid, tm, tn);
    const int m0 = tm * BM;
    const int n0 = tn * BN;
    // GEMM: K is a multiple of 16 (of BK without EDGE); a last partial K tile
    // is completed with zero chunks.  Convolution: the reduction R*S*C is a
    // multiple of 16, completed the same way.
    const int nk = SRC == 0 ? (kslice + BK - 1) / BK : (cv.rsc + BK - 1) / BK;

    // Per-lane source pointers of this wave's load instructions (K offset 0).
    // GEMM: chunks outside the operands read the zero chunk: A rows past M,
    // column-major B rows past N, row-major B columns past N, and chunks at
    // or past K.  One comparison covers all of them: the chunk of slot i in
    // K tile kt exists iff kt * BK < klim[i], with klim[i] = K minus the
    // chunk's K offset within a tile for a row or column that exists, else 0.
    // So only N (row-major B) and K need be multiples of 16 (EDGE forms).
    const int8_t *src[LPW];
    [[maybe_unused]] int klim[LPW];
    // Convolution: per load slot, the row's base (image or filter), the
    // image position of tap (0, 0), the 16-byte chunk of the K tile, and
    // whether the row exists (output pixel < M, output channel < N).
    [[maybe_unused]] int cih[LPW], ciw[LPW], cch[LPW];
    [[maybe_unused]] bool cok[LPW];
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
        const int q = (i * NW + wave) * 64 + lane;
        if constexpr (SRC == 1) {
            const bool is_a = q < A_CHUNKS;
            const int qq = is_a ? q : q - A_CHUNKS;
            const int r = qq / CPR;
            cch[i] = (qq % CPR) ^ chunk_swizzle<CPR>(r);
            if (is_a) {
                const int m = m0 + r;
                cok[i] = m < g.M;
                const int mm = cok[i] ? m : 0;
                const int img = mm / (cv.P * cv.Q);
                const int pq = mm - img * (cv.P * cv.Q);
                const int p = pq / cv.Q;
                const int qc = pq - p * cv.Q;
                cih[i] = p * cv.sh - cv.ph;
                ciw[i] = qc * cv.sw - cv.pw;
                src[i] = g.A + static_cast<int64_t>(img) * cv.H * cv.W * cv.C;
            } else {
                const int n = n0 + r;
                cok[i] = n < g.N;
                cih[i] = ciw[i] = 0;
                src[i] = g.B + static_cast<int64_t>(cok[i] ? n : 0) * g.ldb;
            }
            continue;
        }
        if (q < A_CHUNKS) {
            const int r = q / CPR;
            const int c = (q % CPR) ^ chunk_swizzle<CPR>(r);
            const bool ok = !EDGE || m0 + r < g.M;
            klim[i] = ok ? kslice - 16 * c : 0;
            src[i] = g.A + static_cast<int64_t>(ok ? m0 + r : m0) * g.lda + k_begin + 16 * c;
        } else if constexpr (!BROW) {
            const int qb = q - A_CHUNKS;
            const int r = qb / CPR;
            const int c = (qb % CPR) ^ chunk_swizzle<CPR>(r);
            const bool ok = !EDGE || n0 + r < g.N;
            klim[i] = ok ? kslice - 16 * c : 0;
            src[i] = g.B + static_cast<int64_t>(ok ? n0 + r : n0) * g.ldb + k_begin + 16 * c;
        } else {
            // row-major B: LDS row k of the tile holds B(k0 + k, n0 .. n0+BN-1)
            const int qb = q - A_CHUNKS;
            const int k = qb / CPRB;
            const int c = (qb % CPRB) ^ brow_swizzle<BN>(k);
            const bool ok = !EDGE || n0 + 16 * c < g.N;
            klim[i] = ok ? kslice - k : 0;
            src[i] = g.B + (k_begin + k) * g.ldb + (ok ? n0 + 16 * c : n0);
        }
    }
    // K offset of tile kt for load instruction i.
    auto koff = [&](int i, int kt) -> int64_t {
        const bool is_b = (i * NW + wave) * 64 >= A_CHUNKS;
        return (BROW && is_b) ? static_cast<int64_t>(kt) * BK * g.ldb : static_cast<int64_t>(kt) * BK;
    };
    // Persistent form: the load stream's position (K tile lt of the lj-th
    // tile of this block) and the shifts of the A and B pointers from the
    // first tile to that tile.
    [[maybe_unused]] int lt = 0, lj = 0;
    [[maybe_unused]] int64_t la = 0, lb = 0;
    [[maybe_unused]] const int ptiles =
        PERSIST ? (g.tiles_m * g.tiles_n - static_cast<int>(blockIdx.x) + nblocks - 1) / nblocks : 1;
    // Source of load slot i for K tile kt.
    auto source = [&](int i, int kt) -> const int8_t * {
        if constexpr (PERSIST) {
            const bool is_a = i < A_CHUNKS / 64 / NW;
            return src[i] + (is_a ? la : lb) + koff(i, lt);
        } else if constexpr (SRC == 0 && EDGE) {
            return kt * BK < klim[i] ? src[i] + koff(i, kt) : zero_chunk;
        } else if constexpr (SRC == 0) {
            return src[i] + koff(i, kt);
        } else {
            const bool is_a = (i * NW + wave) * 64 < A_CHUNKS;
            const int kpos = kt * BK + 16 * cch[i];
            if (!cok[i] || kpos >= cv.rsc) return zero_chunk;
            if (!is_a) return src[i] + kpos;
            int c0, r, ss;
            if (cv.tile_in_tap) {
                // The whole K tile lies within one tap: its position (r, s)
                // is the same for every lane (scalar work); a lane adds only
                // its chunk's channel offset.
                const int tap = fast_div(kt * BK, cv.c_div);
                c0 = kt * BK - tap * cv.C + 16 * cch[i];
                r = fast_div(tap, cv.s_div);
                ss = tap - r * cv.S;
            } else {
                const int rs = fast_div(kpos, cv.c_div);
                c0 = kpos - rs * cv.C;
                r = fast_div(rs, cv.s_div);
                ss = rs - r * cv.S;
            }
            const int ih = cih[i] + r * cv.dh;
            const int iw = ciw[i] + ss * cv.dw;
            if (static_cast<unsigned>(ih) >= static_cast<unsigned>(cv.H) ||
                static_cast<unsigned>(iw) >= static_cast<unsigned>(cv.W))
                return zero_chunk;
            return src[i] + (static_cast<int64_t>(ih) * cv.W + iw) * cv.C + c0;
        }
    };
    // One block row over M: each B byte is read by one block only, so B
    // streams past the cache and leaves it to A (row-major skinny column
    // groups, the 16x16x64 split forms: 4-5%).  Compiled into those forms
    // only: the run-time test cost the 256 x 256 kernel 1%.
    const bool b_once = SRC == 0 && SPLIT && MF == 16 && g.tiles_m == 1;
    auto issue_one = [&](int kt, int i) {
        int8_t *dst = lds + (kt % STAGES) * STAGE + (i * NW + wave) * 1024;
        if (b_once && (i * NW + wave) * 64 >= A_CHUNKS)
            __builtin_amdgcn_global_load_lds(source(i, kt), (lds_void_t *)dst, 16, 0, kLoadStream);
        else
            __builtin_amdgcn_global_load_lds(source(i, kt), (lds_void_t *)dst, 16, 0, 0);
    };
    auto issue = [&](int kt) {
#pragma unroll
        for (int i = 0; i < LPW; ++i) issue_one(kt, i);
    };
    // Persistent form: the stream moves on by one K tile (all of its load
    // slots issued); past a tile's last one it moves to the block's next
    // tile.
    auto advance = [&]() {
        if constexpr (PERSIST) {
            if (++lt == nk) {
                lt = 0;
                if (++lj < ptiles) {
                    int tm2, tn2;
                    tile_of_block(g, static_cast<int>(blockIdx.x) + lj * nblocks, tm2, tn2);
                    la = static_cast<int64_t>(tm2 * BM - m0) * g.lda;
                    lb = BROW ? static_cast<int64_t>(tn2 * BN - n0) : static_cast<int64_t>(tn2 * BN - n0) * g.ldb;
                }
            }
        }
    };

    // LDS byte offsets (within a stage) of this lane's operand rows.
    const int lrow = lane % MF;
    const int lgrp = lane / MF;
    int offa[MT], offb[NT], swa[MT], swb[NT];
#pragma unroll
    for (int i = 0; i < MT; ++i) {
        const int r = wm * (MT * MF) + i * MF + lrow;
        offa[i] = r * BK;
        swa[i] = chunk_swizzle<CPR>(r);
    }
#pragma unroll
    for (int j = 0; j < NT; ++j) {
        const int r = BM + wn * (NT * MF) + j * MF + lrow;
        offb[j] = r * BK;
        swb[j] = chunk_swizzle<CPR>(r - BM);
    }

    // Row-major B operands come from two transpose reads per fragment
    // (brow_frag_offsets).
    int offbt[NT][2];
    if constexpr (BROW) {
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            brow_frag_offsets<MF, BN>(lane, wn * (NT * MF) + j * MF, offbt[j][0], offbt[j][1]);
            offbt[j][0] += A_BYTES_;
            offbt[j][1] += A_BYTES_;
        }
    }

    Acc acc[MT][NT];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NT; ++j) acc[i][j] = Acc{};

    // Operand registers: [buffer][K step of the group][fragment].
    i32x4 fa[2][G][MT], fb[2][G][NT];
    constexpr int F1 = MT * NT;  // matrix-core instructions per K step
    constexpr int R1 = MT + NT;  // operand reads per K step
    // Read rr of group gi of tile kt (K step gi * G + rr / R1, fragment rr % R1).
    auto read_one = [&](int kt, int gi, int buf, int rr) {
        const int s = rr / R1, r = rr % R1;
        const int ks = gi * G + s;
        const int8_t *base = lds + (kt % STAGES) * STAGE;
        const int c = ks * KC + lgrp;
        if (r < MT) {
            fa[buf][s][r] = *reinterpret_cast<const i32x4 *>(base + offa[r] + 16 * (c ^ swa[r]));
        } else if constexpr (!BROW) {
            fb[buf][s][r - MT] = *reinterpret_cast<const i32x4 *>(base + offb[r - MT] + 16 * (c ^ swb[r - MT]));
        } else {
            fb[buf][s][r - MT] = read_tr_frag(base + offbt[r - MT][0] + ks * KSTEP * BN,
                                              base + offbt[r - MT][1] + ks * KSTEP * BN);
        }
    };
    constexpr int F = G * F1;    // matrix-core instructions per group
    constexpr int R = G * R1;    // operand reads per group
    auto read_frags = [&](int kt, int gi, int buf) {
#pragma unroll
        for (int rr = 0; rr < R; ++rr) read_one(kt, gi, buf, rr);
    };
    auto mma_one = [&](int buf, int x) {
        const int s = x / F1, i = (x % F1) / NT, j = x % NT;
        acc[i][j] = Mfma<MF>::run(fb[buf][s][j], fa[buf][s][i], acc[i][j]);
    };
    // Read r of a group is issued after matrix instruction r / 2: two per
    // instruction, at the front of the group, so the last one has most of the
    // group to land before the group's closing wait.  Row-major B, whose
    // fragments are two transpose reads each, spreads them one fragment per
    // instruction (16384^2 x 8192: 2049 -> 2015 us; with column-major B that
    // spacing measured 1806 -> 1819 us, so it keeps two).
    auto read_slot = [](int r) constexpr -> int {
        const int x = BROW ? r : r / 2;
        return x < F ? x : F - 1;
    };

    // One K tile, as a fixed instruction order (each matrix-core instruction
    // followed by the memory operations slotted after it, fenced so the
    // compiler keeps the order):
    //  * groups 0 .. KG-2: matrix work of the group, with the operand reads
    //    of the next group slotted in (read_slot);
    //  * last group: its operands are already in registers, so first publish
    //    tile t+1 (own DMA loads of t+1 retired, then a barrier: every wave
    //    is done with buffer t % STAGES), refill that buffer with tile
    //    t+STAGES, then the group's matrix work with tile t+1's first-group
    //    operands read in between.
    // Every group ends by retiring its operand reads, so the next group's
    // matrix work starts with its operands in registers.  Issuing a refill
    // right after the barrier that frees its buffer gives it the longest
    // possible time in flight (a whole K tile with two stages).
    //   LOAD:  issue tile t+STAGES after the barrier;
    //   NEXT:  tile t+1 exists (barrier, next-tile reads);
    //   WAITN: the loads of tiles t+2 .. t+STAGES-1 are in flight and may
    //          stay so; otherwise wait for every outstanding load.
    auto tile = [&](int t, auto load_tag, auto next_tag, auto waitn_tag) {
        constexpr bool LOAD = decltype(load_tag)::value;
        constexpr bool NEXT = decltype(next_tag)::value;
        constexpr bool WAITN = decltype(waitn_tag)::value;
#pragma unroll
        for (int gi = 0; gi < KG; ++gi) {
            const int cur = gi & 1;
            if (gi + 1 < KG) {
#pragma unroll
                for (int x = 0; x < F; ++x) {
                    mma_one(cur, x);
#pragma unroll
                    for (int r = 0; r < R; ++r)
                        if (read_slot(r) == x) read_one(t, gi + 1, cur ^ 1, r);
                    __builtin_amdgcn_sched_barrier(0);
                }
            } else {
                if constexpr (NEXT) {
                    if constexpr (WAITN) {
                        TDI8_WAIT_VMCNT((STAGES - 2) * LPW);
                    } else {
                        TDI8_WAIT_VMCNT(0);
                    }
                    TDI8_WAIT_LGKM0();
                    block_barrier();
                    __builtin_amdgcn_sched_barrier(0);
                }
                // Row-major B: the refill goes out at once.  Column-major B:
                // spread over the step's matrix instructions (measured 2%
                // faster at 16384^2 x 8192, 7% slower with row-major B).
                if constexpr (LOAD && BROW) {
                    issue(t + STAGES);
                    advance();
                    __builtin_amdgcn_sched_barrier(0);
                }
#pragma unroll
                for (int x = 0; x < F; ++x) {
                    if constexpr (LOAD && !BROW) {
#pragma unroll
                        for (int li = 0; li < LPW; ++li)
                            if ((li * F) / LPW == x) issue_one(t + STAGES, li);
                    }
                    mma_one(cur, x);
                    if constexpr (NEXT) {
#pragma unroll
                        for (int r = 0; r < R; ++r)
                            if (read_slot(r) == x) read_one(t + 1, 0, cur ^ 1, r);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
                if constexpr (LOAD && !BROW) advance();
            }
            TDI8_WAIT_LGKM0();
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    using T1 = std::true_type;
    using T0 = std::false_type;

    if constexpr (PERSIST) {
        // The tile's C straight from the accumulation registers, each store
        // instruction writing whole 128-byte lines with the non-temporal
        // hint.  Lane l = 32 h + r of an instruction tile holds, in its
        // quads q = 0..3, row r's 16-byte pieces 2 q + h (columns
        // 8 q + 4 h .. + 3).  Two lane exchanges regroup them: swapping
        // 16-lane rows between quads 0/1 and 2/3 (v_permlane16_swap) puts
        // rows 0..15 in quads 0 and 2 and rows 16..31 in quads 1 and 3, then
        // swapping lanes 8 apart between quads 0/2 and 1/3 (DPP row_ror:8)
        // leaves, for lane l = 32 h + 16 s + 8 t + k, row k (+8, +16, +24 in
        // quads 2, 1, 3) piece 4 t + 2 s + h in every quad: one instruction
        // per quad covers 8 rows x 128 bytes.
        auto store_tile = [&](int j) {
            int tm2, tn2;
            tile_of_block(g, static_cast<int>(blockIdx.x) + j * nblocks, tm2, tn2);
            const int k8 = lane & 7;
            const bool t8 = (lane >> 3) & 1;
            const int piece = 4 * (t8 ? 1 : 0) + 2 * ((lane >> 4) & 1) + (lane >> 5);
            int32_t *cb = g.C + static_cast<int64_t>(tm2 * BM + wm * (MT * MF) + k8) * g.ldc + tn2 * BN +
                          wn * (NT * MF) + 4 * piece;
            constexpr int kRowOf[4] = {0, 16, 8, 24};  // first row held by quad 0, 1, 2, 3
#pragma unroll
            for (int i = 0; i < MT; ++i)
#pragma unroll
                for (int jj = 0; jj < NT; ++jj) {
                    int q[4][4];
#pragma unroll
                    for (int qq = 0; qq < 4; ++qq)
#pragma unroll
                        for (int e = 0; e < 4; ++e) q[qq][e] = acc[i][jj][4 * qq + e];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
#pragma unroll
                        for (int pq = 0; pq < 4; pq += 2) {
                            const auto r = __builtin_amdgcn_permlane16_swap(q[pq][e], q[pq + 1][e], false, false);
                            q[pq][e] = static_cast<int>(r[0]);
                            q[pq + 1][e] = static_cast<int>(r[1]);
                        }
#pragma unroll
                        for (int pq = 0; pq < 2; ++pq) {
                            const int lo = __builtin_amdgcn_update_dpp(0, q[pq][e], 0x128, 0xf, 0xf, false);
                            const int hi = __builtin_amdgcn_update_dpp(0, q[pq + 2][e], 0x128, 0xf, 0xf, false);
                            q[pq][e] = t8 ? hi : q[pq][e];
                            q[pq + 2][e] = t8 ? q[pq + 2][e] : lo;
                        }
                    }
#pragma unroll
                    for (int qq = 0; qq < 4; ++qq) {
                        const i32x4 v = {q[qq][0], q[qq][1], q[qq][2], q[qq][3]};
                        __builtin_nontemporal_store(
                            v, reinterpret_cast<i32x4 *>(cb + static_cast<int64_t>(i * MF + kRowOf[qq]) * g.ldc + jj * MF));
                    }
                }
        };
        int ct = 0, cj = 0;  // K tile within the tile being computed, and that tile's index
        // After each K tile of the stream: a tile whose last K tile is done
        // is stored, and the accumulators start over for the next one.
        auto finish = [&]() {
            if (++ct == nk) {
                ct = 0;
                store_tile(cj++);
#pragma unroll
                for (int i = 0; i < MT; ++i)
#pragma unroll
                    for (int j = 0; j < NT; ++j) acc[i][j] = Acc{};
            }
        };
        const int total = ptiles * nk;
        if (total > 0) {
            const int first = total < STAGES ? total : STAGES;
            for (int s = 0; s < first; ++s) {
                issue(s);
                advance();
            }
            if (total >= STAGES) {
                TDI8_WAIT_VMCNT((STAGES - 1) * LPW);
            } else {
                TDI8_WAIT_VMCNT(0);
            }
            block_barrier();
            read_frags(0, 0, 0);
            TDI8_WAIT_LGKM0();
            __builtin_amdgcn_sched_barrier(0);
            int u = 0;
            for (; u + STAGES < total; ++u) {
                tile(u, T1{}, T1{}, T1{});
                finish();
            }
            if (u + STAGES == total && u + 1 < total) {
                tile(u, T0{}, T1{}, T1{});
                finish();
                ++u;
            }
            for (; u + 1 < total; ++u) {
                tile(u, T0{}, T1{}, T0{});
                finish();
            }
            tile(u, T0{}, T0{}, T0{});
            stamp.loop_done();
            finish();
        } else {
            // K = 0: every tile of the block is zero.
            stamp.loop_done();
            for (int j = 0; j < ptiles; ++j) store_tile(j);
        }
        stamp.end(g);
        return;
    }

    if (nk > 0) {
        // Prologue: every buffer filled (tiles 0 .. STAGES-1), wait for tile 0.
        if (nk >= STAGES) {
#pragma unroll
            for (int s = 0; s < STAGES; ++s) issue(s);
            TDI8_WAIT_VMCNT((STAGES - 1) * LPW);
        } else {
            for (int s = 0; s < nk; ++s) issue(s);
            TDI8_WAIT_VMCNT(0);
        }
        block_barrier();
        read_frags(0, 0, 0);
        TDI8_WAIT_LGKM0();  // the K loop starts with no operand read pending
        __builtin_amdgcn_sched_barrier(0);

        int t = 0;
        // Steady state: every iteration refills the buffer it frees.
        for (; t + STAGES < nk; ++t) tile(t, T1{}, T1{}, T1{});
        // Last refill was issued one iteration ago: tiles t+2 .. nk-1 in flight.
        if (t + STAGES == nk && t + 1 < nk) {
            tile(t, T0{}, T1{}, T1{});
            ++t;
        }
        // Drain: wait for everything outstanding.
        for (; t + 1 < nk; ++t) tile(t, T0{}, T1{}, T0{});
        tile(t, T0{}, T0{}, T0{});
    }
    stamp.loop_done();

    if constexpr (SPLIT) {
        // Partial sums go through LDS (free once the K loop is done), so that
        // each atomic instruction covers 64 consecutive columns of one row
        // (two cache lines) instead of 32 rows.  Rows of the tile are taken
        // in passes of RP (a multiple of the 32-row instruction tile) that fit
        // the stage buffers with a 16-byte pad per row (the pad keeps the
        // 32 rows written by one instruction on different banks).
        constexpr int LDS_TOTAL = STAGES * STAGE;
        constexpr int RS = BN + 4;                                  // int32 per LDS row
        constexpr int RP0 = (LDS_TOTAL / (RS * 4)) / MF * MF;
        constexpr int RP = RP0 < BM ? RP0 : BM;
        static_assert(RP >= MF, "stage buffers hold at least one instruction tile of rows");
        int32_t *cl = reinterpret_cast<int32_t *>(lds);
        for (int p0 = 0; p0 < BM; p0 += RP) {
            __syncthreads();
#pragma unroll
            for (int i = 0; i < MT; ++i) {
                const int rb = wm * (MT * MF) + i * MF;  // first tile row of this instruction tile
                if (rb < p0 || rb >= p0 + RP) continue;
#pragma unroll
                for (int j = 0; j < NT; ++j) {
                    const int cb = wn * (NT * MF) + j * MF;
                    if constexpr (MF == 32) {
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            const int r = rb - p0 + (lane & 31);
                            const int c = cb + 8 * q + 4 * (lane >> 5);
                            *reinterpret_cast<i32x4 *>(cl + r * RS + c) =
                                i32x4{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
                        }
                    } else {
                        *reinterpret_cast<i32x4 *>(cl + (rb - p0 + (lane & 15)) * RS + cb + 4 * (lane >> 4)) = acc[i][j];
                    }
                }
            }
            __syncthreads();
            const int rows = BM - p0 < RP ? BM - p0 : RP;
            for (int idx = threadIdx.x; idx < rows * BN; idx += NW * 64) {
                const int r = idx / BN;
                const int c = idx - r * BN;
                if (!EDGE || (m0 + p0 + r < g.M && n0 + c < g.N))
                    atomicAdd(g.C + static_cast<int64_t>(m0 + p0 + r) * g.ldc + n0 + c, cl[r * RS + c]);
            }
        }
        stamp.end(g);
        return;
    }

    const bool full_rows = !EDGE || (m0 + BM <= g.M && n0 + BN <= g.N);  // the whole tile exists
    if constexpr (MF == 32) {
        // C through LDS (free once the K loop is done), in passes of RP rows
        // as in the split epilogue: a store instruction then covers 64
        // consecutive 16-byte pieces of whole rows instead of 32 rows x 32
        // bytes, so every 128-byte line is written whole by one instruction
        // and the stores can carry the non-temporal hint (C is not read
        // again here; it then stops evicting the A and B lines other blocks
        // still use).  Measured against the per-lane stores: 4096^3 3%
        // (row-major B 11%), 8192^2 x 4096 6% (11%), 2048^3 24%.  Hinted
        // stores of 32-byte pieces were 36% slower instead.
        constexpr int LDS_TOTAL = STAGES * STAGE;
        constexpr int RS = BN + 4;
        constexpr int RP0 = (LDS_TOTAL / (RS * 4)) / MF * MF;
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
            for (int idx = threadIdx.x; idx < rows * (BN / 4); idx += NW * 64) {
                const int r = idx / (BN / 4);
                const int c4 = idx - r * (BN / 4);
                const i32x4 v = *reinterpret_cast<const i32x4 *>(cl + r * RS + 4 * c4);
                if (SRC == 0 && full_rows)
                    store4_nt<true>(g, m0 + p0 + r, n0 + 4 * c4, v);
                else
                    store4_nt<false>(g, m0 + p0 + r, n0 + 4 * c4, v);
            }
        }
    } else {
        // 16x16 instruction tiles: lane holds C[m][n .. n+3], stored directly.
#pragma unroll
        for (int i = 0; i < MT; ++i) {
#pragma unroll
            for (int j = 0; j < NT; ++j) {
                const int mb = m0 + wm * (MT * MF) + i * MF;
                const int nb = n0 + wn * (NT * MF) + j * MF;
                if (SRC == 0 && full_rows)
                    store4<true>(g, mb + (lane & 15), nb + 4 * (lane >> 4), acc[i][j]);
                else
                    store4<false>(g, mb + (lane & 15), nb + 4 * (lane >> 4), acc[i][j]);
            }
        }
    }
    stamp.end(g);
#endif
}

template <int MF, int WM, int WN, int MT, int NT, int BK, int STAGES, bool BROW, bool SPLIT, bool EDGE>
__global__ void __launch_bounds__(WM * WN * 64) gemm_rc_pipelined_kernel(GemmArgs g) {
    pipelined_body<MF, WM, WN, MT, NT, BK, STAGES, BROW, SPLIT, EDGE, 0>(g, ConvParams{});
}

// Persistent form of the whole-tile kernel: nblocks blocks (at most the tile
// count; a multiple of 8 keeps each block on one XCD) walk all tiles, see
// PERSIST above.
template <int MF, int WM, int WN, int MT, int NT, int BK, int STAGES, bool BROW>
__global__ void __launch_bounds__(WM * WN * 64) gemm_rc_persistent_kernel(GemmArgs g, int nblocks) {
    pipelined_body<MF, WM, WN, MT, NT, BK, STAGES, BROW, false, false, 0, true>(g, ConvParams{}, nblocks);
}

// Implicit-GEMM convolution ("先导杯比赛回顾", 卷积转化: the convolution
// lowered to a matrix product, here without materialising the im2col
// matrix): A row m = output pixel (n, p, q) of an NHWC image, A column
// (r, s, c) = the input byte the im2col index map picks, B = the KRSC filter
// bank read as a column-major K x (R S C) matrix, C = the N P Q x K output.
// Every 16-byte A chunk is 16 channels of one tap, gathered straight into LDS
// by the same DMA loads; taps outside the image, the K tail past R S C and
// rows past M or N read a zero chunk instead.
template <int MF, int WM, int WN, int MT, int NT, int BK, int STAGES>
__global__ void __launch_bounds__(WM * WN * 64) conv_implicit_kernel(GemmArgs g, ConvParams cv) {
    pipelined_body<MF, WM, WN, MT, NT, BK, STAGES, false, false, true, 1>(g, cv);
}

}  // namespace tdi8
