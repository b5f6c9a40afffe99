// C ABI entry points: argument checks, per-device initialisation, selection
// and kernel launch.  The pages' launchers print the HIP error after each
// launch (contest write-up, the NCHW_2_NHWC and Im2col launch wrappers); a
// library returns it instead.
#include <hip/hip_runtime.h>

#include <climits>
#include <cstdint>
#include <cstring>
#include <mutex>

#include "../../include/tdi8.h"
#if defined(TDI8_STAMPS)
#include "../../include/tdi8_stamps.h"
#endif
#include "kernel_table.h"
#include "selector.h"
#include "device_common.h"

namespace tdi8 {

// C[0:M, 0:N] = 0 (C 16-byte aligned, ldc a multiple of 4; a row's last
// group of four may be partial): run before a K-split launch, whose blocks
// add their partial sums into C.
__global__ void __launch_bounds__(256) zero_c_kernel(GemmArgs g) {
    const int64_t per_row = (g.N + 3) / 4;
    const int64_t total = per_row * g.M;
    for (int64_t q = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; q < total;
         q += static_cast<int64_t>(gridDim.x) * 256) {
        const int64_t m = q / per_row;
        const int64_t n = 4 * (q - m * per_row);
        int32_t *p = g.C + m * g.ldc + n;
        if (n + 4 <= g.N) {
            *reinterpret_cast<i32x4 *>(p) = i32x4{0, 0, 0, 0};
        } else {
            for (int j = 0; j < g.N - n; ++j) p[j] = 0;
        }
    }
}

namespace {

thread_local int g_last_hip_error = 0;

int hip_fail(hipError_t e) {
    g_last_hip_error = static_cast<int>(e);
    return TDI8_ERR_HIP;
}

#if defined(TDI8_STAMPS)
// Timeline buffer of the instrumented library (tdi8_stamps_set).
uint64_t *g_stamps = nullptr;
int g_stamp_cap = 0;
void attach_stamps(GemmArgs &g) {
    g.stamps = g_stamps;
    g.stamp_cap = g_stamp_cap;
}
#else
void attach_stamps(GemmArgs &) {}
#endif

const KernelSet *kernels() {
    static const KernelSet *table = [] {
        static KernelSet ks[TDI8_NUM_CONFIGS];
#define TDI8_CALL_REGISTER(ID, ...) register_cfg_##ID(&ks[ID]);
        TDI8_CONFIG_LIST(TDI8_CALL_REGISTER)
#undef TDI8_CALL_REGISTER
        return ks;
    }();
    return table;
}

constexpr int kMaxDevices = 64;

struct DeviceState {
    std::once_flag once;
    int status = TDI8_OK;
    int hip_error = 0;
    tdi8_hw_info hw{};
    int bpc[TDI8_NUM_CONFIGS] = {};
    // resident blocks per compute unit of each persistent kernel [config][b_col_major]
    // (its registers can differ from the one-tile-per-block kernel's)
    int persist_bpc[TDI8_NUM_CONFIGS][2] = {};
};

DeviceState g_devices[kMaxDevices];

void init_device(DeviceState &ds, int dev) {
    hipDeviceProp_t prop;
    hipError_t e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) {
        ds.status = TDI8_ERR_HIP;
        ds.hip_error = static_cast<int>(e);
        return;
    }
    if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0) {
        ds.status = TDI8_ERR_UNSUPPORTED_DEVICE;
        return;
    }
    ds.hw.num_cu = prop.multiProcessorCount;
    ds.hw.max_threads_per_block = prop.maxThreadsPerBlock;
    ds.hw.min_active_threads = 4 * prop.warpSize;  // one wave on each of the 4 SIMDs of a CU
    ds.hw.skinny_max_m = 32;
    for (int id = 0; id < TDI8_NUM_CONFIGS; ++id) {
        const StaticCfg c = static_cfg(id);
        const void *k = kernels()[id].kernel[1][1];
        int nb = 0;
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, k, c.threads, 0);
        if (e != hipSuccess) {
            ds.status = TDI8_ERR_HIP;
            ds.hip_error = static_cast<int>(e);
            return;
        }
        ds.bpc[id] = nb;
        for (int b = 0; b < 2; ++b) {
            const void *pk = kernels()[id].persist[b];
            if (!pk) continue;
            e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, pk, c.threads, 0);
            if (e != hipSuccess) {
                ds.status = TDI8_ERR_HIP;
                ds.hip_error = static_cast<int>(e);
                return;
            }
            ds.persist_bpc[id][b] = nb;
        }
    }
}

// Initialised state of the current device, or nullptr with *status set.
DeviceState *current_device(int *status) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) {
        *status = hip_fail(e);
        return nullptr;
    }
    if (dev < 0 || dev >= kMaxDevices) {
        *status = TDI8_ERR_UNSUPPORTED_DEVICE;
        return nullptr;
    }
    DeviceState &ds = g_devices[dev];
    std::call_once(ds.once, [&] { init_device(ds, dev); });
    if (ds.status != TDI8_OK) {
        if (ds.status == TDI8_ERR_HIP) g_last_hip_error = ds.hip_error;
        *status = ds.status;
        return nullptr;
    }
    return &ds;
}

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Which kernel runs a call, on which grid: one decision, shared by the launch
// and the gemm_plan query, so that what the query reports is what runs.
struct Plan {
    int form = TDI8_FORM_NONE;
    const void *kernel = nullptr;
    bool zero_first = false;  // a fill kernel zeroes the C window first (K split)
    dim3 grid, block;
    GemmArgs g{};
    int nblocks = 0;          // persistent form: its block count, the kernel's second argument
};

int make_plan(int id, int bcol, int M, int N, int K, const int8_t *A, int lda, const int8_t *B, int ldb,
              int32_t *C, int ldc, int num_cu, Plan *p) {
    const StaticCfg c = static_cfg(id);
    GemmArgs &g = p->g;
    g.splits = 1;
    g.A = A;
    g.B = B;
    g.C = C;
    g.lda = lda;
    g.ldb = ldb;
    g.ldc = ldc;
    g.M = M;
    g.N = N;
    g.K = K;
    const int b = bcol ? 1 : 0;
    const bool c_ok = aligned(C, 16) && ldc % 4 == 0;
    const bool a_ok = aligned(A, 16) && lda % 16 == 0;
    const bool b_ok = aligned(B, 16) && ldb % 16 == 0;
    p->block = dim3(c.threads);
    if (c.family == 0) {
        const int64_t tm = (M + static_cast<int64_t>(c.bm) - 1) / c.bm;
        const int64_t tn = (N + static_cast<int64_t>(c.bn) - 1) / c.bn;
        if (tm * tn > INT_MAX / c.threads) return TDI8_ERR_INVALID_VALUE;
        g.tiles_m = static_cast<int>(tm);
        g.tiles_n = static_cast<int>(tn);
        // both B layouts are moved by 16-byte LDS DMA loads in the fast form;
        // chunks outside the operands read a zero chunk and stores are
        // masked, so M and N are free and K (and, row-major B, N) need only
        // be multiples of 16 (the edge form: sizes that end inside a tile);
        // the K split runs in the whole-tile form when M, N and every slice
        // are whole tiles, else in the edge form (slices of 16-byte chunks)
        const bool fast = K % 16 == 0 && (bcol || N % 16 == 0) && a_ok && b_ok && c_ok;
        const bool edge = fast && (M % c.bm != 0 || N % c.bn != 0 || K % c.bk != 0);
        if (fast) g.splits = split_k_for(c, M, N, K, num_cu);
        if (g.splits > 1) {
            const bool whole = !edge && K % (g.splits * c.bk) == 0;
            p->form = whole ? TDI8_FORM_SPLIT : TDI8_FORM_SPLIT_EDGE;
            p->kernel = whole ? kernels()[id].split[b] : kernels()[id].split_edge[b];
            p->zero_first = true;
            p->grid = dim3(static_cast<unsigned>(tm * tn * g.splits));
        } else {
            p->form = !fast ? TDI8_FORM_PREDICATED : edge ? TDI8_FORM_PIPELINED_EDGE : TDI8_FORM_PIPELINED;
            p->kernel = edge ? kernels()[id].edge[b] : kernels()[id].kernel[b][fast ? 1 : 0];
            p->grid = dim3(static_cast<unsigned>(tm * tn));
            // The predicated kernel with two K tiles of loads in flight pays
            // when each compute unit holds at most one block, whose loop is
            // then latency-bound (1000 x 1000 x 8191: 80.8 -> 49.9 us); with
            // more blocks per unit, whose loads already keep its
            // misaligned-load path busy, it cost 3-13% (1000 x 3000 x 777:
            // 12.2 -> 13.8 us).  It needs column-major B, K >= 16 and
            // three K tiles.
            if (!fast && bcol && kernels()[id].prefetch && tm * tn <= num_cu && K >= 16 &&
                (K + c.bk - 1) / c.bk >= 3) {
                p->form = TDI8_FORM_PREDICATED_PREFETCH;
                p->kernel = kernels()[id].prefetch;
            }
        }
        return TDI8_OK;
    }
    // Skinny family.  The unpredicated forms move B by 16-byte LDS DMA loads
    // in both layouts; a ragged M (M < 16 included) reads zero chunks past M,
    // and a last, partial K chunk zero pieces past K (K a multiple of 16).
    const bool dma_ok = a_ok && b_ok && c_ok;
    const bool fast = N % c.bn == 0 && K % 16 == 0 && dma_ok;
    // Row-major B: the column-group form (kernel_table.h) when N and K are
    // whole 16-byte chunks (the edge form: a last group may end inside its
    // 128 columns, a K slice inside a K tile; the last slices may be
    // shorter) and N is whole groups or more than two of them (a narrow N
    // would leave most of every group's columns empty: 4096 x 16 x 4096 took
    // 29 us that way against 6 in the per-tile form).
    const int groups = kRrGroupCols / c.bn;
    if (!bcol && dma_ok && (N % kRrGroupCols == 0 || N > 2 * kRrGroupCols) && N % 16 == 0 && K % 16 == 0) {
        const int64_t tm = (M + static_cast<int64_t>(c.bm) - 1) / c.bm;
        const int64_t tn = (N + kRrGroupCols - 1) / kRrGroupCols;
        if (tm * tn * groups <= INT_MAX / 512) {
            g.tiles_m = static_cast<int>(tm);
            g.tiles_n = static_cast<int>(tn);
            g.splits = groups;
            p->form = TDI8_FORM_SKINNY_ROW_GROUPS;
            p->kernel = kernels()[id].rr_group;
            p->zero_first = true;
            p->grid = dim3(static_cast<unsigned>(tm * tn * groups));
            p->block = dim3(512);
            return TDI8_OK;
        }
    }
    // the predicated row-major form covers 64 columns per block
    const int bn = (bcol || fast) ? c.bn : 64;
    const int64_t tm = (M + static_cast<int64_t>(c.bm) - 1) / c.bm;
    const int64_t tn = (N + static_cast<int64_t>(bn) - 1) / bn;
    if (tm > 65535) return TDI8_ERR_BAD_CONFIG;
    if (tn > INT_MAX / c.threads) return TDI8_ERR_INVALID_VALUE;
    g.tiles_m = static_cast<int>(tm);
    g.tiles_n = static_cast<int>(tn);
    p->form = fast ? TDI8_FORM_SKINNY_DMA : TDI8_FORM_SKINNY_PREDICATED;
    p->kernel = kernels()[id].kernel[b][fast ? 1 : 0];
    p->grid = dim3(static_cast<unsigned>(tn), static_cast<unsigned>(tm));
    return TDI8_OK;
}

// Enqueue a plan: for a K split, first the fill kernel that zeroes the C
// window, whose blocks then add their partial sums into it.
int run_plan(Plan &p, hipStream_t stream) {
    attach_stamps(p.g);
    void *args[] = {&p.g};
    void *pargs[] = {&p.g, &p.nblocks};  // the persistent kernel's two arguments
    hipError_t e;
    if (p.zero_first) {
        const int64_t quads = static_cast<int64_t>(p.g.M) * ((p.g.N + 3) / 4);
        const unsigned zb = static_cast<unsigned>(quads / 256 + 1 < 2048 ? quads / 256 + 1 : 2048);
        e = hipLaunchKernel(reinterpret_cast<const void *>(&zero_c_kernel), dim3(zb), dim3(256), args, 0, stream);
        if (e != hipSuccess) return hip_fail(e);
    }
    e = hipLaunchKernel(p.kernel, p.grid, p.block, p.form == TDI8_FORM_PERSISTENT ? pargs : args, 0, stream);
    if (e != hipSuccess) return hip_fail(e);
    return TDI8_OK;
}

bool overlaps(uintptr_t a0, uintptr_t a1, uintptr_t b0, uintptr_t b1) { return a0 < b1 && b0 < a1; }

// The plan of a call: the given configuration, or (cfg -1) the selection's,
// with the predicated column-major form moved to a configuration whose tiles
// fill more compute units when the selected ones leave some idle
// (predicated_fill; 1000 x 1000 x 8191 with a tight odd leading dimension:
// 64 x 128 tiles, 128 blocks, 50.2 us; 64 x 64 tiles, 256 blocks, 35.4 us).
int plan_call(int cfg, int bcol, int M, int N, int K, const int8_t *A, int lda, const int8_t *B, int ldb,
              int32_t *C, int ldc, const DeviceState &ds, Plan *p, int *id_out) {
    int id = cfg;
    if (id < 0) {
        id = select_config(M, N, K, ds.hw, ds.bpc, nullptr);
        if (id < 0) return id;
    }
    int st = make_plan(id, bcol, M, N, K, A, lda, B, ldb, C, ldc, ds.hw.num_cu, p);
    if (st != TDI8_OK) return st;
    if (cfg < 0 && bcol && (p->form == TDI8_FORM_PREDICATED || p->form == TDI8_FORM_PREDICATED_PREFETCH)) {
        const int fill = predicated_fill(id, M, N, ds.hw.num_cu);
        if (fill != id) {
            id = fill;
            *p = Plan{};
            st = make_plan(id, bcol, M, N, K, A, lda, B, ldb, C, ldc, ds.hw.num_cu, p);
            if (st != TDI8_OK) return st;
        }
    }
    *id_out = id;
    return TDI8_OK;
}

int gemm_entry(int cfg, int bcol, int M, int N, int K, const int8_t *A, int lda, const int8_t *B, int ldb,
               int32_t *C, int ldc, hipStream_t stream) {
    int st = tdi8_validate(bcol, M, N, K, A, lda, B, ldb, C, ldc);
    if (st != TDI8_OK) return st;
    if (cfg >= TDI8_NUM_CONFIGS || cfg < -1) return TDI8_ERR_BAD_CONFIG;
    if (M == 0 || N == 0) return TDI8_OK;
    DeviceState *ds = current_device(&st);
    if (!ds) return st;
    Plan p;
    int id = -1;
    st = plan_call(cfg, bcol, M, N, K, A, lda, B, ldb, C, ldc, *ds, &p, &id);
    if (st != TDI8_OK) return st;
    return run_plan(p, stream);
}

// The persistent form of configuration id (general family) over whole tiles;
// blocks 0 = one wave of resident blocks of the persistent kernel itself (its
// occupancy, not the one-tile kernel's), rounded down to a multiple of 8.
int persistent_entry(int cfg, int bcol, int M, int N, int K, const int8_t *A, int lda, const int8_t *B, int ldb,
                     int32_t *C, int ldc, int blocks, hipStream_t stream) {
    int st = tdi8_validate(bcol, M, N, K, A, lda, B, ldb, C, ldc);
    if (st != TDI8_OK) return st;
    if (cfg >= TDI8_NUM_CONFIGS || cfg < -1) return TDI8_ERR_BAD_CONFIG;
    if (blocks < 0) return TDI8_ERR_INVALID_VALUE;
    if (M == 0 || N == 0) return TDI8_OK;
    DeviceState *ds = current_device(&st);
    if (!ds) return st;
    const int id = cfg < 0 ? select_config(M, N, K, ds->hw, ds->bpc, nullptr) : cfg;
    if (id < 0) return id;
    const StaticCfg c = static_cfg(id);
    if (c.family != 0) return TDI8_ERR_BAD_CONFIG;
    const bool whole = M % c.bm == 0 && N % c.bn == 0 && K % c.bk == 0;
    const bool al = aligned(A, 16) && lda % 16 == 0 && aligned(B, 16) && ldb % 16 == 0 && aligned(C, 16) &&
                    ldc % 4 == 0;
    if (!whole || !al) return TDI8_ERR_BAD_CONFIG;
    const int64_t tiles = static_cast<int64_t>(M / c.bm) * (N / c.bn);
    if (tiles > INT_MAX / c.threads) return TDI8_ERR_INVALID_VALUE;
    int64_t nb = blocks;
    if (nb == 0) {
        const int pb = ds->persist_bpc[id][bcol ? 1 : 0];
        nb = static_cast<int64_t>(ds->hw.num_cu) * (pb > 0 ? pb : 1);
        if (nb >= 8) nb -= nb % 8;
    }
    if (nb > tiles) nb = tiles;
    Plan p;
    p.form = TDI8_FORM_PERSISTENT;
    p.kernel = kernels()[id].persist[bcol ? 1 : 0];
    p.block = dim3(c.threads);
    p.grid = dim3(static_cast<unsigned>(nb));
    p.nblocks = static_cast<int>(nb);
    GemmArgs &g = p.g;
    g.A = A;
    g.B = B;
    g.C = C;
    g.lda = lda;
    g.ldb = ldb;
    g.ldc = ldc;
    g.M = M;
    g.N = N;
    g.K = K;
    g.tiles_m = M / c.bm;
    g.tiles_n = N / c.bn;
    g.splits = 1;
    return run_plan(p, stream);
}

int64_t conv_extent(int64_t H, int64_t R, int64_t pad, int64_t stride, int64_t dil) {
    const int64_t span = H + 2 * pad - dil * (R - 1) - 1;
    return span < 0 ? 0 : span / stride + 1;
}

struct ConvShape {
    int N, H, W, C, K, R, S, ph, pw, sh, sw, dh, dw;
};

// Host checks of a convolution call; fills the GEMM view and the geometry.
int conv_check(const ConvShape &c, const int8_t *x, const int8_t *w, const int32_t *y, GemmArgs *g,
               ConvParams *cv) {
    if (c.N < 0 || c.H < 0 || c.W < 0 || c.C < 0 || c.K < 0 || c.R < 1 || c.S < 1 || c.ph < 0 || c.pw < 0 ||
        c.sh < 1 || c.sw < 1 || c.dh < 1 || c.dw < 1)
        return TDI8_ERR_INVALID_VALUE;
    const int64_t P = conv_extent(c.H, c.R, c.ph, c.sh, c.dh);
    const int64_t Q = conv_extent(c.W, c.S, c.pw, c.sw, c.dw);
    const int64_t M = static_cast<int64_t>(c.N) * P * Q;
    const int64_t rsc = static_cast<int64_t>(c.R) * c.S * c.C;
    if (M > INT_MAX || rsc > INT_MAX || P > INT_MAX || Q > INT_MAX) return TDI8_ERR_INVALID_VALUE;
    g->A = x;
    g->B = w;
    g->C = const_cast<int32_t *>(y);
    g->lda = 0;
    g->ldb = rsc;
    g->ldc = c.K;
    g->M = static_cast<int>(M);
    g->N = c.K;
    g->K = static_cast<int>(rsc);
    g->splits = 1;
    *cv = ConvParams{c.N, c.H, c.W, c.C, c.R, c.S, static_cast<int>(P), static_cast<int>(Q),
                     c.sh, c.sw, c.ph, c.pw, c.dh, c.dw, static_cast<int>(rsc),
                     make_fast_div(c.C > 0 ? c.C : 1), make_fast_div(c.S), 0, 0, 1, make_fast_div(1)};
    if (M == 0 || c.K == 0) return TDI8_OK;
    if (!y) return TDI8_ERR_NULL_POINTER;
    if (!aligned(y, 4)) return TDI8_ERR_INVALID_VALUE;
    if (rsc == 0) return TDI8_OK;
    if (!x || !w) return TDI8_ERR_NULL_POINTER;
    const uintptr_t y0 = reinterpret_cast<uintptr_t>(y);
    const uintptr_t y1 = y0 + 4 * static_cast<uint64_t>(M) * static_cast<uint64_t>(c.K);
    const uintptr_t x0 = reinterpret_cast<uintptr_t>(x);
    const uintptr_t x1 = x0 + static_cast<uint64_t>(c.N) * c.H * c.W * c.C;
    const uintptr_t w0 = reinterpret_cast<uintptr_t>(w);
    const uintptr_t w1 = w0 + static_cast<uint64_t>(c.K) * static_cast<uint64_t>(rsc);
    if (overlaps(y0, y1, x0, x1) || overlaps(y0, y1, w0, w1)) return TDI8_ERR_ALIASING;
    return TDI8_OK;
}

int conv_entry(int cfg, const ConvShape &c, const int8_t *x, const int8_t *w, int32_t *y, hipStream_t stream) {
    GemmArgs g;
    ConvParams cv;
    int st = conv_check(c, x, w, y, &g, &cv);
    if (st != TDI8_OK) return st;
    if (cfg >= TDI8_NUM_CONFIGS || cfg < -1) return TDI8_ERR_BAD_CONFIG;
    if (g.M == 0 || g.N == 0) return TDI8_OK;
    DeviceState *ds = current_device(&st);
    if (!ds) return st;
    int id = cfg;
    if (id < 0) {
        tdi8_hw_info hw = ds->hw;
        hw.skinny_max_m = 0;  // the convolution form exists for the general family only
        id = select_config(g.M, g.N, g.K, hw, ds->bpc, nullptr);
        if (id < 0) return id;
    }
    const StaticCfg sc = static_cfg(id);
    if (sc.family != 0) return TDI8_ERR_BAD_CONFIG;
    const int64_t tm = (g.M + static_cast<int64_t>(sc.bm) - 1) / sc.bm;
    const int64_t tn = (g.N + static_cast<int64_t>(sc.bn) - 1) / sc.bn;
    if (tm * tn > INT_MAX / sc.threads) return TDI8_ERR_INVALID_VALUE;
    g.tiles_m = static_cast<int>(tm);
    g.tiles_n = static_cast<int>(tn);
    // 16-byte DMA chunks are 16 channels of one tap: C a multiple of 16 and
    // 16-byte aligned operands; otherwise the gather form.
    const bool dma = c.C % 16 == 0 && aligned(x, 16) && aligned(w, 16);
    cv.tile_in_tap = dma && c.C % sc.bk == 0;
    // gather form without horizontal dilation: the run form (conv_run16),
    // whose reduction is R filter rows of ceil(S C / 16) 16-byte pieces
    if (!dma && c.dw == 1) {
        const int64_t run = static_cast<int64_t>(c.S) * c.C;
        const int64_t runp = (run + 15) / 16;
        if (c.R * runp * 16 <= INT_MAX) {
            cv.run = static_cast<int>(run);
            cv.runp = static_cast<int>(runp);
            cv.runp_div = make_fast_div(cv.runp);
            g.K = static_cast<int>(c.R * runp * 16);
        }
    }
    attach_stamps(g);
    void *args[] = {&g, &cv};
    hipError_t e = hipLaunchKernel(dma ? kernels()[id].conv : kernels()[id].conv_gather,
                                   dim3(static_cast<unsigned>(tm * tn)), dim3(sc.threads), args, 0, stream);
    if (e != hipSuccess) return hip_fail(e);
    return TDI8_OK;
}

}  // namespace
}  // namespace tdi8

using namespace tdi8;

extern "C" {

int tdi8_validate(int b_col_major, int M, int N, int K, const int8_t *A, int lda, const int8_t *B, int ldb,
                  const int32_t *C, int ldc) {
    if (M < 0 || N < 0 || K < 0) return TDI8_ERR_INVALID_VALUE;
    const int kmin = K > 1 ? K : 1;
    const int nmin = N > 1 ? N : 1;
    if (lda < kmin || ldc < nmin || ldb < (b_col_major ? kmin : nmin)) return TDI8_ERR_INVALID_VALUE;
    if (M == 0 || N == 0) return TDI8_OK;
    if (!C) return TDI8_ERR_NULL_POINTER;
    if (K == 0) return TDI8_OK;
    if (!A || !B) return TDI8_ERR_NULL_POINTER;
    const uintptr_t c0 = reinterpret_cast<uintptr_t>(C);
    const uintptr_t c1 = c0 + 4 * (static_cast<uint64_t>(M - 1) * static_cast<uint64_t>(ldc) + N);
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(A);
    const uintptr_t a1 = a0 + static_cast<uint64_t>(M - 1) * static_cast<uint64_t>(lda) + K;
    const uintptr_t b0 = reinterpret_cast<uintptr_t>(B);
    const uintptr_t b1 = b0 + (b_col_major ? static_cast<uint64_t>(N - 1) * static_cast<uint64_t>(ldb) + K
                                           : static_cast<uint64_t>(K - 1) * static_cast<uint64_t>(ldb) + N);
    if (overlaps(c0, c1, a0, a1) || overlaps(c0, c1, b0, b1)) return TDI8_ERR_ALIASING;
    return TDI8_OK;
}

int gemm_s8s8s32(int M, int N, int K, const int8_t *A, int lda, const int8_t *B, int ldb, int32_t *C, int ldc,
                 hipStream_t stream) {
    return gemm_entry(-1, 0, M, N, K, A, lda, B, ldb, C, ldc, stream);
}

int gemm_s8s8s32_bt(int M, int N, int K, const int8_t *A, int lda, const int8_t *B, int ldb, int32_t *C, int ldc,
                    hipStream_t stream) {
    return gemm_entry(-1, 1, M, N, K, A, lda, B, ldb, C, ldc, stream);
}

int gemm_s8s8s32_with_config(int config_id, int b_col_major, int M, int N, int K, const int8_t *A, int lda,
                             const int8_t *B, int ldb, int32_t *C, int ldc, hipStream_t stream) {
    if (config_id < 0 || config_id >= TDI8_NUM_CONFIGS) return TDI8_ERR_BAD_CONFIG;
    return gemm_entry(config_id, b_col_major ? 1 : 0, M, N, K, A, lda, B, ldb, C, ldc, stream);
}

int gemm_s8s8s32_persistent(int config_id, int b_col_major, int M, int N, int K, const int8_t *A, int lda,
                            const int8_t *B, int ldb, int32_t *C, int ldc, int blocks, hipStream_t stream) {
    return persistent_entry(config_id, b_col_major ? 1 : 0, M, N, K, A, lda, B, ldb, C, ldc, blocks, stream);
}

int select_tile_config(int M, int N, int K) {
    if (M < 0 || N < 0 || K < 0) return TDI8_ERR_INVALID_VALUE;
    int st = TDI8_OK;
    DeviceState *ds = current_device(&st);
    if (!ds) return st;
    return select_config(M, N, K, ds->hw, ds->bpc, nullptr);
}

int select_tile_config_for(int M, int N, int K, const tdi8_hw_info *hw, const int *blocks_per_cu,
                           tdi8_selection *out) {
    if (M < 0 || N < 0 || K < 0) return TDI8_ERR_INVALID_VALUE;
    if (!hw || !blocks_per_cu) return TDI8_ERR_NULL_POINTER;
    if (hw->num_cu <= 0 || hw->max_threads_per_block <= 0) return TDI8_ERR_INVALID_VALUE;
    return select_config(M, N, K, *hw, blocks_per_cu, out);
}

int tile_config_count(void) { return TDI8_NUM_CONFIGS; }

int conv2d_output_extent(int H, int R, int pad, int stride, int dil) {
    if (H < 0 || R < 1 || pad < 0 || stride < 1 || dil < 1) return TDI8_ERR_INVALID_VALUE;
    const int64_t e = conv_extent(H, R, pad, stride, dil);
    return e > INT_MAX ? TDI8_ERR_INVALID_VALUE : static_cast<int>(e);
}

int conv2d_validate(int N, int H, int W, int C, int K, int R, int S, int pad_h, int pad_w, int stride_h,
                    int stride_w, int dil_h, int dil_w, const int8_t *x, const int8_t *w, const int32_t *y) {
    GemmArgs g;
    ConvParams cv;
    return conv_check(ConvShape{N, H, W, C, K, R, S, pad_h, pad_w, stride_h, stride_w, dil_h, dil_w}, x, w, y,
                      &g, &cv);
}

int conv2d_s8s8s32_nhwc(int N, int H, int W, int C, int K, int R, int S, int pad_h, int pad_w, int stride_h,
                        int stride_w, int dil_h, int dil_w, const int8_t *x, const int8_t *w, int32_t *y,
                        hipStream_t stream) {
    return conv_entry(-1, ConvShape{N, H, W, C, K, R, S, pad_h, pad_w, stride_h, stride_w, dil_h, dil_w}, x, w,
                      y, stream);
}

int conv2d_s8s8s32_nhwc_with_config(int config_id, int N, int H, int W, int C, int K, int R, int S, int pad_h,
                                    int pad_w, int stride_h, int stride_w, int dil_h, int dil_w, const int8_t *x,
                                    const int8_t *w, int32_t *y, hipStream_t stream) {
    if (config_id < 0 || config_id >= TDI8_NUM_CONFIGS) return TDI8_ERR_BAD_CONFIG;
    return conv_entry(config_id, ConvShape{N, H, W, C, K, R, S, pad_h, pad_w, stride_h, stride_w, dil_h, dil_w},
                      x, w, y, stream);
}

int conv2d_select_config(int N, int H, int W, int C, int K, int R, int S, int pad_h, int pad_w, int stride_h,
                         int stride_w, int dil_h, int dil_w) {
    GemmArgs g;
    ConvParams cv;
    const int st = conv_check(ConvShape{N, H, W, C, K, R, S, pad_h, pad_w, stride_h, stride_w, dil_h, dil_w},
                              nullptr, nullptr, nullptr, &g, &cv);
    if (st != TDI8_OK && st != TDI8_ERR_NULL_POINTER) return st;
    int s2 = TDI8_OK;
    DeviceState *ds = current_device(&s2);
    if (!ds) return s2;
    tdi8_hw_info hw = ds->hw;
    hw.skinny_max_m = 0;
    return select_config(g.M, g.N, g.K, hw, ds->bpc, nullptr);
}

int tile_config_split_k(int config_id, int M, int N, int K, int num_cu) {
    if (config_id < 0 || config_id >= TDI8_NUM_CONFIGS) return TDI8_ERR_BAD_CONFIG;
    if (M < 0 || N < 0 || K < 0 || num_cu <= 0) return TDI8_ERR_INVALID_VALUE;
    return split_k_for(static_cfg(config_id), M, N, K, num_cu);
}

int tile_config_info(int id, tdi8_tile_config *out) {
    if (id < 0 || id >= TDI8_NUM_CONFIGS) return TDI8_ERR_BAD_CONFIG;
    if (!out) return TDI8_ERR_NULL_POINTER;
    const StaticCfg c = static_cfg(id);
    const KernelResources &r = kKernelResources[id];
    tdi8_tile_config t{};
    t.id = id;
    t.family = c.family;
    t.mfma_m = c.mf;
    t.mfma_n = c.mf;
    t.mfma_k = c.mfma_k;
    t.waves_m = c.wm;
    t.waves_n = c.wn;
    t.waves_k = c.wk;
    t.m_tiles = c.mt;
    t.n_tiles = c.nt;
    t.block_m = c.bm;
    t.block_n = c.bn;
    t.block_k = c.bk;
    t.stages = c.stages;
    t.threads = c.threads;
    t.lds_bytes = r.lds_bytes;
    t.vgprs = r.unified_vgprs - r.agprs;
    t.agprs = r.agprs;
    t.sgprs = r.sgprs;
    t.reuse1_id = c.reuse1_id;
    t.excluded = c.excluded;
    int dev = -1;
    if (hipGetDevice(&dev) == hipSuccess && dev >= 0 && dev < kMaxDevices) {
        int st = TDI8_OK;
        DeviceState *ds = current_device(&st);
        if (ds) t.blocks_per_cu = ds->bpc[id];
    }
    *out = t;
    return TDI8_OK;
}

int gemm_plan(int config_id, int b_col_major, int M, int N, int K, const int8_t *A, int lda, const int8_t *B,
              int ldb, const int32_t *C, int ldc, tdi8_plan *out) {
    if (!out) return TDI8_ERR_NULL_POINTER;
    if (config_id < -1 || config_id >= TDI8_NUM_CONFIGS) return TDI8_ERR_BAD_CONFIG;
    const int bcol = b_col_major ? 1 : 0;
    int st = tdi8_validate(bcol, M, N, K, A, lda, B, ldb, C, ldc);
    if (st != TDI8_OK) return st;
    tdi8_plan r{};
    r.config_id = config_id;
    r.form = TDI8_FORM_NONE;
    if (M == 0 || N == 0) {
        *out = r;
        return TDI8_OK;
    }
    DeviceState *ds = current_device(&st);
    if (!ds) return st;
    Plan p;
    int id = -1;
    st = plan_call(config_id, bcol, M, N, K, A, lda, B, ldb, const_cast<int32_t *>(C), ldc, *ds, &p, &id);
    if (st != TDI8_OK) return st;
    r.config_id = id;
    r.form = p.form;
    r.splits = p.g.splits;
    r.kernels = p.zero_first ? 2 : 1;
    r.grid_x = static_cast<int>(p.grid.x);
    r.grid_y = static_cast<int>(p.grid.y);
    r.threads = static_cast<int>(p.block.x);
    *out = r;
    return TDI8_OK;
}

const char *tdi8_status_string(int status) {
    switch (status) {
        case TDI8_OK: return "ok";
        case TDI8_ERR_INVALID_VALUE: return "invalid value (negative size or leading dimension too small)";
        case TDI8_ERR_NULL_POINTER: return "null pointer";
        case TDI8_ERR_ALIASING: return "C overlaps A or B";
        case TDI8_ERR_UNSUPPORTED_DEVICE: return "unsupported device (gfx950 required)";
        case TDI8_ERR_BAD_CONFIG: return "bad configuration id for this shape";
        case TDI8_ERR_HIP: return "HIP runtime error";
        default: return "unknown status";
    }
}

int tdi8_last_hip_error(void) { return g_last_hip_error; }

#if defined(TDI8_STAMPS)
int tdi8_stamps_set(uint64_t *records, int capacity) {
    if (capacity < 0 || (capacity > 0 && records == nullptr)) return TDI8_ERR_INVALID_VALUE;
    g_stamps = capacity > 0 ? records : nullptr;
    g_stamp_cap = capacity;
    return TDI8_OK;
}
#endif

}  // extern "C"
