// Host-side selection of a tile configuration (no HIP dependency).
#pragma once

#include "../../include/tdi8.h"
#include "configs.h"

namespace tdi8 {

// Static parameters of one configuration, derived from the configuration list.
struct StaticCfg {
    int id, family, mf, wm, wn, wk, mt, nt, bk, stages;
    int block_m_threads, block_n_threads;  // the claims' thread split along M and N
    int bm, bn;                            // block tile
    int threads, mfma_k, lds_bytes;
    int reuse1_id;                         // same split with m_tiles = n_tiles = 1, or -1
    int excluded;                          // reuse scheme excluded by claim 3's performance test
};

StaticCfg static_cfg(int id);

// Configuration that runs a selected general configuration when the call
// takes the predicated form with column-major B: the selection counts on the
// K split to fill the compute units when its tiles are few, which the
// predicated kernels cannot do, so when the selected tiles number fewer than
// num_cu, the reuse-1 general configuration with the most tiles (at most
// num_cu; ties to the deeper K tile, then table order) runs instead, if it
// has more tiles.  A CDNA4 rule after the five steps, not one of them.
int predicated_fill(int id, int M, int N, int num_cu);

// The selection on described hardware; bpc[id] = resident blocks per compute
// unit of configuration id.  Returns the id, or a negative status.
int select_config(int M, int N, int K, const tdi8_hw_info &hw, const int *bpc, tdi8_selection *out);

// K slices for the unpredicated form of a general configuration (a CDNA4
// addition after the five steps; split K with integer atomics, the contest
// write-up's "Split K" paragraph): K a multiple of 16, tiles counted with
// the partial ones at M's and N's ends; while the tiles times twice the
// slices still fit one block per compute unit, and K over twice the slices
// is still at least eight K tiles, the slices double (slices of four to
// seven K tiles measured up to 18% slower than half as many of twice the
// length).  1 = no split.
int split_k_for(const StaticCfg &c, int M, int N, int K, int num_cu);

}  // namespace tdi8
