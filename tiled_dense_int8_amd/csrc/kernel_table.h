// Host-side view of the compiled configurations: static parameters from the
// configuration list and the kernel entry points of each one.
#pragma once

#include "configs.h"

namespace tdi8 {

template <int ID>
struct CfgParams;

#define TDI8_DEFINE_PARAMS(ID, FAM, MF_, WM_, WN_, WK_, MT_, NT_, BK_, ST_)              \
    template <>                                                                          \
    struct CfgParams<ID> {                                                               \
        static constexpr int family = FAM, mf = MF_, wm = WM_, wn = WN_, wk = WK_,       \
                             mt = MT_, nt = NT_, bk = BK_, st = ST_;                     \
    };
TDI8_CONFIG_LIST(TDI8_DEFINE_PARAMS)
#undef TDI8_DEFINE_PARAMS

// kernel[b_col_major][fast]: host stubs of the four instantiations (the fast
// general kernel for whole tiles); split[b_col_major]: its K-split form,
// edge[b_col_major]: its form for sizes that end inside a tile and
// split_edge[b_col_major]: the K split of that form, whose slices may end
// inside a K tile (null for the skinny family); prefetch: the predicated
// column-major-B kernel with the deep-prefetch K loop (null where the tile
// does not fit it, and for the skinny family); conv: the implicit-GEMM
// convolution form; persist[b_col_major]: the persistent form of the
// whole-tile kernel (general family; null for the skinny family).
struct KernelSet {
    const void *kernel[2][2];
    const void *persist[2];
    const void *prefetch;
    const void *split[2];
    const void *edge[2];
    const void *split_edge[2];
    const void *conv;   // implicit-GEMM convolution form (null for the skinny family)
    const void *conv_gather;  // its gather form: any channel count or alignment
    const void *rr_group;  // row-major B column-group form (skinny family only)
};

// Row-major B column-group form of a skinny configuration (BM x BN tile):
// one block covers BM x kRrGroupCols outputs over 1/G of K, G = kRrGroupCols
// / BN, so the grid keeps the configuration's block count while every B row
// segment a block reads is a whole 128-byte line; the G partial sums of a
// tile are added into a zeroed C.  K tile of the form per block height:
constexpr int kRrGroupCols = 128;
constexpr int rr_group_bk(int bm) { return bm == 16 ? 512 : 256; }

// Resources of a configuration's column-major-B unpredicated kernel
// (kernel[1][1], the one its occupancy is taken on), read by the build from
// the AMDGPU metadata of the compiled code object: vector registers per lane
// (the metadata's count, which on gfx950 spans both register files: the
// architectural registers, rounded up to a multiple of 4, then the
// accumulation registers), of which accumulation registers, scalar registers
// per wave, static LDS per block and scratch per lane in bytes.
struct KernelResources {
    int unified_vgprs, agprs, sgprs, lds_bytes, scratch_bytes;
};
extern const KernelResources kKernelResources[TDI8_NUM_CONFIGS];

// One registration function per configuration, each defined in its own
// translation unit so the instantiations compile in parallel.
#define TDI8_DECLARE_REGISTER(ID, ...) void register_cfg_##ID(KernelSet *ks);
TDI8_CONFIG_LIST(TDI8_DECLARE_REGISTER)
#undef TDI8_DECLARE_REGISTER

}  // namespace tdi8
