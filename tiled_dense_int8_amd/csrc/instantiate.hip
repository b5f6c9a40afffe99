// Instantiates the kernels of configuration TDI8_CFG (set on the compiler
// command line, one object per configuration) and registers their entry
// points.  Patent application CN114238853A, claim 7: every configuration's
// parameters become the kernel's template parameters and all are compiled.
#include "kernel_table.h"
#include "rc_pipelined_kernel.h"
#include "skinny_kernel.h"
#include "tiled_kernel.h"

#ifndef TDI8_CFG
#error "TDI8_CFG must name a configuration id"
#endif

#define TDI8_CAT2(a, b) a##b
#define TDI8_CAT(a, b) TDI8_CAT2(a, b)

namespace tdi8 {

// Pipeline depth of the unpredicated kernel per B layout.  A configuration's
// stage count is its column-major kernel's; with row-major B the 64 x 128
// and 128 x 64 tiles keep two stages, since there three resident blocks per
// compute unit (instead of two) gain more than the deeper prefetch
// (512x4096x4096: 29.7 against 31.5 us; 1024x1024x8192: 41.8 against 46.1).
template <class P, bool BCOL>
constexpr int stages_for() {
    return BCOL || P::st < 3 ? P::st : 2;
}

template <class P, bool BCOL, bool FAST>
static const void *entry() {
    if constexpr (P::family == 0 && FAST)
        return reinterpret_cast<const void *>(
            &gemm_rc_pipelined_kernel<P::mf, P::wm, P::wn, P::mt, P::nt, P::bk, stages_for<P, BCOL>(), !BCOL, false,
                                      false>);
    else if constexpr (P::family == 0)
        return reinterpret_cast<const void *>(
            &gemm_tiled_kernel<P::mf, P::wm, P::wn, P::mt, P::nt, P::bk, BCOL, FAST>);
    else if constexpr (BCOL && FAST)
        return reinterpret_cast<const void *>(&gemm_skinny_lds_kernel<P::mt, P::nt, P::wk, P::bk>);
    else if constexpr (BCOL)
        return reinterpret_cast<const void *>(&gemm_skinny_kernel<P::mt, P::nt, P::wk, P::st, false>);
    else if constexpr (FAST)
        return reinterpret_cast<const void *>(&gemm_skinny_rrlds_kernel<P::mt, P::nt, P::wk, P::bk>);
    else
        return reinterpret_cast<const void *>(&gemm_skinny_rr_kernel<P::mt, P::wk, 2, false>);
}

template <class P, bool BCOL>
static const void *split_entry() {
    if constexpr (P::family == 0)
        return reinterpret_cast<const void *>(
            &gemm_rc_pipelined_kernel<P::mf, P::wm, P::wn, P::mt, P::nt, P::bk, stages_for<P, BCOL>(), !BCOL, true,
                                      false>);
    else
        return nullptr;
}

// Persistent form of the whole-tile general kernel.
template <class P, bool BCOL>
static const void *persist_entry() {
    if constexpr (P::family == 0)
        return reinterpret_cast<const void *>(
            &gemm_rc_persistent_kernel<P::mf, P::wm, P::wn, P::mt, P::nt, P::bk, stages_for<P, BCOL>(), !BCOL>);
    else
        return nullptr;
}

// The unpredicated general kernel for sizes that end inside a tile.
template <class P, bool BCOL>
static const void *edge_entry() {
    if constexpr (P::family == 0)
        return reinterpret_cast<const void *>(
            &gemm_rc_pipelined_kernel<P::mf, P::wm, P::wn, P::mt, P::nt, P::bk, stages_for<P, BCOL>(), !BCOL, false,
                                      true>);
    else
        return nullptr;
}

// Its K-split form (slices of 16-byte chunks).
template <class P, bool BCOL>
static const void *split_edge_entry() {
    if constexpr (P::family == 0)
        return reinterpret_cast<const void *>(
            &gemm_rc_pipelined_kernel<P::mf, P::wm, P::wn, P::mt, P::nt, P::bk, stages_for<P, BCOL>(), !BCOL, true,
                                      true>);
    else
        return nullptr;
}

// The predicated column-major-B kernel with the deep-prefetch loop, for
// tiles that fit it.
template <class P>
static const void *prefetch_entry() {
    if constexpr (P::family == 0 &&
                  deep_prefetch_fits(P::wm * P::mf * P::mt, P::wn * P::mf * P::nt, P::bk, P::wm * P::wn * 64))
        return reinterpret_cast<const void *>(&gemm_tiled_prefetch_kernel<P::mf, P::wm, P::wn, P::mt, P::nt, P::bk>);
    else
        return nullptr;
}

template <class P>
static const void *conv_entry() {
    if constexpr (P::family == 0)
        return reinterpret_cast<const void *>(&conv_implicit_kernel<P::mf, P::wm, P::wn, P::mt, P::nt, P::bk, P::st>);
    else
        return nullptr;
}

template <class P>
static const void *conv_gather_entry() {
    if constexpr (P::family == 0)
        return reinterpret_cast<const void *>(&conv_gather_kernel<P::mf, P::wm, P::wn, P::mt, P::nt, P::bk>);
    else
        return nullptr;
}

// Row-major B column-group form of the skinny family: 8 waves, one per
// 16-column slice of the 128-column group; 16 rows (one instruction tile,
// K tile 512, two stages) or 32 rows (two instruction tiles, K tile 256,
// three stages).
template <class P>
static const void *rr_group_entry() {
    if constexpr (P::family == 1 && P::mt == 1) {
        static_assert(rr_group_bk(16) == 512, "K tile of the 16-row form");
        return reinterpret_cast<const void *>(&gemm_rc_pipelined_kernel<16, 1, 8, 1, 1, 512, 2, true, true, true>);
    } else if constexpr (P::family == 1 && P::mt == 2) {
        static_assert(rr_group_bk(32) == 256, "K tile of the 32-row form");
        return reinterpret_cast<const void *>(&gemm_rc_pipelined_kernel<16, 1, 8, 2, 1, 256, 3, true, true, true>);
    } else {
        return nullptr;
    }
}

void TDI8_CAT(register_cfg_, TDI8_CFG)(KernelSet *ks) {
    using P = CfgParams<TDI8_CFG>;
    ks->kernel[0][0] = entry<P, false, false>();
    ks->kernel[0][1] = entry<P, false, true>();
    ks->kernel[1][0] = entry<P, true, false>();
    ks->kernel[1][1] = entry<P, true, true>();
    ks->persist[0] = persist_entry<P, false>();
    ks->persist[1] = persist_entry<P, true>();
    ks->prefetch = prefetch_entry<P>();
    ks->split[0] = split_entry<P, false>();
    ks->split[1] = split_entry<P, true>();
    ks->edge[0] = edge_entry<P, false>();
    ks->edge[1] = edge_entry<P, true>();
    ks->split_edge[0] = split_edge_entry<P, false>();
    ks->split_edge[1] = split_edge_entry<P, true>();
    ks->conv = conv_entry<P>();
    ks->conv_gather = conv_gather_entry<P>();
    ks->rr_group = rr_group_entry<P>();
}

}  // namespace tdi8
