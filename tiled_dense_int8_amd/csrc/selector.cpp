// Tile-configuration selection: the five steps of patent application
// CN114238853A claim 1, with claims 2-6 read for CDNA4.  Host-only, no HIP.
//
//  step 1  the candidates are the compiled configurations (claim 7);
//  step 2  thread split along M and N: multiples of the matrix-core tile,
//          each at least 16, at most max_threads_per_block threads (claim 2,
//          matrix-unit case); drop configurations whose register-limited
//          active threads per compute unit, blocks_per_cu * threads, stay
//          below the threshold (claim 3, first alternative) and those whose
//          reuse scheme the performance test excluded (claim 3, second
//          alternative: TDI8_EXCLUDED_REUSE in configs.h);
//  step 3  Thread_Blocks = ceil(M / BM) * ceil(N / BN) must reach
//          min_theory_block_num = num_cu * blocks_per_cu; if no configuration
//          does, the size is too small to fill the compute units and every
//          step-2 survivor is reduced to reuse 1 (m_tiles = n_tiles = 1: its
//          reuse-1 sibling) and kept (claim 4).  For M <= skinny_max_m the
//          candidates then become the skinny family with the smallest block
//          height >= M (else, for N <= skinny_max_m, with the smallest block
//          width >= N), keeping those with at least one block per compute
//          unit (all of them if none has) and of these the smallest block
//          width (block height);
//  step 4  keep the largest compute-to-memory ratio of a K step,
//          BM*BN*BK / (BM*BK + BK*BN) = BM*BN / (BM + BN), compared exactly
//          by cross-multiplication (claim 5; the B tile width uses n_tiles);
//  step 5  keep the fewest kernel rounds ceil(Thread_Blocks / (num_cu *
//          blocks_per_cu)) (claim 6); remaining ties go to table order.
#include "selector.h"

#include <cstdint>

namespace tdi8 {

namespace {

struct Desc {
    int id, family, mf, wm, wn, wk, mt, nt, bk, st;
};

constexpr Desc kDesc[] = {
#define TDI8_DESC(ID, FAM, MF, WM, WN, WK, MT, NT, BK, ST) {ID, FAM, MF, WM, WN, WK, MT, NT, BK, ST},
    TDI8_CONFIG_LIST(TDI8_DESC)
#undef TDI8_DESC
};

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace

StaticCfg static_cfg(int id) {
    const Desc &d = kDesc[id];
    StaticCfg s{};
    s.id = d.id;
    s.family = d.family;
    s.mf = d.mf;
    s.wm = d.wm;
    s.wn = d.wn;
    s.wk = d.wk;
    s.mt = d.mt;
    s.nt = d.nt;
    s.bk = d.bk;
    s.stages = d.st;
    s.block_m_threads = d.wm * d.mf;
    s.block_n_threads = d.wn * d.mf;
    s.bm = s.block_m_threads * d.mt;
    s.bn = s.block_n_threads * d.nt;
    s.threads = 64 * d.wm * d.wn * d.wk;
    s.mfma_k = d.mf == 32 ? 32 : 64;
    s.lds_bytes = d.family == 0 ? d.st * (s.bm + s.bn) * d.bk
                                : 2 * (s.bm + s.bn) * (d.bk + 16) + d.mt * d.nt * 64 * 16;
    s.excluded = 0;
#define TDI8_EXCLUDE(FAM, MT, NT) \
    if (d.family == (FAM) && d.mt == (MT) && d.nt == (NT)) s.excluded = 1;
    TDI8_EXCLUDED_REUSE(TDI8_EXCLUDE)
#undef TDI8_EXCLUDE
    s.reuse1_id = -1;
    for (const Desc &e : kDesc) {
        if (e.family == d.family && e.mf == d.mf && e.wm == d.wm && e.wn == d.wn && e.wk == d.wk &&
            e.bk == d.bk && e.mt == 1 && e.nt == 1) {
            s.reuse1_id = e.id;
            break;
        }
    }
    return s;
}

namespace {

struct Cand {
    StaticCfg c;
    int bpc;
};

int64_t thread_blocks(const StaticCfg &c, int64_t M, int64_t N) { return cdiv(M, c.bm) * cdiv(N, c.bn); }

bool passes_step2(const StaticCfg &c, int bpc, const tdi8_hw_info &hw) {
    const bool split = c.block_m_threads % c.mf == 0 && c.block_n_threads % c.mf == 0 &&
                       c.block_m_threads >= 16 && c.block_n_threads >= 16 &&
                       c.threads <= hw.max_threads_per_block;
    return !c.excluded && split && bpc >= 1 && static_cast<int64_t>(bpc) * c.threads >= hw.min_active_threads;
}

// Sign of ratio(a) - ratio(b) with ratio = BM*BN/(BM+BN).
int compare_ratio(const StaticCfg &a, const StaticCfg &b) {
    const int64_t l = static_cast<int64_t>(a.bm) * a.bn * (b.bm + b.bn);
    const int64_t r = static_cast<int64_t>(b.bm) * b.bn * (a.bm + a.bn);
    return (l > r) - (l < r);
}

}  // namespace

int select_config(int M, int N, int K, const tdi8_hw_info &hw, const int *bpc, tdi8_selection *out) {
    (void)K;  // the claims select on (m, n) only
    Cand list[TDI8_NUM_CONFIGS];
    int count[5] = {0, 0, 0, 0, 0};

    // Step 1: the general configurations whose block tile does not overhang
    // the problem (block height at most max(M, smallest height in the list),
    // width likewise; a CDNA4 addition: a larger block only adds zero rows
    // or columns), or all of them if none qualifies.  Then step 2.
    int min_bm = 0, min_bn = 0;
    for (int id = 0; id < TDI8_NUM_CONFIGS; ++id) {
        const StaticCfg c = static_cfg(id);
        if (c.family != 0) continue;
        if (min_bm == 0 || c.bm < min_bm) min_bm = c.bm;
        if (min_bn == 0 || c.bn < min_bn) min_bn = c.bn;
    }
    auto fits = [&](const StaticCfg &c) {
        return c.bm <= (M > min_bm ? M : min_bm) && c.bn <= (N > min_bn ? N : min_bn);
    };
    bool any_fit = false;
    for (int id = 0; id < TDI8_NUM_CONFIGS; ++id) {
        const StaticCfg c = static_cfg(id);
        if (c.family == 0 && fits(c)) any_fit = true;
    }
    Cand s2[TDI8_NUM_CONFIGS];
    int n2 = 0;
    for (int id = 0; id < TDI8_NUM_CONFIGS; ++id) {
        const StaticCfg c = static_cfg(id);
        if (c.family != 0 || (any_fit && !fits(c))) continue;
        ++count[0];
        if (passes_step2(c, bpc[id], hw)) s2[n2++] = Cand{c, bpc[id]};
    }
    count[1] = n2;
    if (n2 == 0) return TDI8_ERR_BAD_CONFIG;

    // Step 3.
    int n3 = 0;
    int route = TDI8_ROUTE_GENERAL;
    for (int i = 0; i < n2; ++i)
        if (thread_blocks(s2[i].c, M, N) >= static_cast<int64_t>(hw.num_cu) * s2[i].bpc) list[n3++] = s2[i];
    if (n3 == 0) {
        route = TDI8_ROUTE_FALLBACK;
        bool taken[TDI8_NUM_CONFIGS] = {};
        for (int i = 0; i < n2; ++i) {
            const int r = s2[i].c.reuse1_id;
            if (r >= 0 && !taken[r] && passes_step2(static_cfg(r), bpc[r], hw)) taken[r] = true;
        }
        bool sib_fit = false;
        for (int id = 0; id < TDI8_NUM_CONFIGS; ++id)
            if (taken[id] && fits(static_cfg(id))) sib_fit = true;
        for (int id = 0; id < TDI8_NUM_CONFIGS; ++id)
            if (taken[id] && (!sib_fit || fits(static_cfg(id)))) list[n3++] = Cand{static_cfg(id), bpc[id]};
        // The skinny family covers a small M, or else a small N: its block
        // extent along that dimension is the smallest one >= it.
        const bool by_m = M <= hw.skinny_max_m;
        if (by_m || N <= hw.skinny_max_m) {
            const int small = by_m ? M : N;
            auto extent = [&](const StaticCfg &c) { return by_m ? c.bm : c.bn; };
            int best_ext = 0;
            for (int id = 0; id < TDI8_NUM_CONFIGS; ++id) {
                const StaticCfg c = static_cfg(id);
                if (c.family == 1 && extent(c) >= small && passes_step2(c, bpc[id], hw) &&
                    (best_ext == 0 || extent(c) < best_ext))
                    best_ext = extent(c);
            }
            if (best_ext > 0) {
                route = TDI8_ROUTE_SKINNY;
                Cand sk[TDI8_NUM_CONFIGS];
                int nsk = 0, nfill = 0;
                for (int id = 0; id < TDI8_NUM_CONFIGS; ++id) {
                    const StaticCfg c = static_cfg(id);
                    if (c.family == 1 && extent(c) == best_ext && passes_step2(c, bpc[id], hw))
                        sk[nsk++] = Cand{c, bpc[id]};
                }
                for (int i = 0; i < nsk; ++i)
                    if (thread_blocks(sk[i].c, M, N) >= hw.num_cu) list[nfill++] = sk[i];
                if (nfill == 0)
                    for (int i = 0; i < nsk; ++i) list[nfill++] = sk[i];
                // of those, the smallest extent along the other dimension:
                // the most blocks, each streaming its share of the large
                // operand
                auto other = [&](const StaticCfg &c) { return by_m ? c.bn : c.bm; };
                int least = 0;
                for (int i = 0; i < nfill; ++i)
                    if (least == 0 || other(list[i].c) < least) least = other(list[i].c);
                n3 = 0;
                for (int i = 0; i < nfill; ++i)
                    if (other(list[i].c) == least) list[n3++] = list[i];
            }
        }
    }
    count[2] = n3;

    // Step 4: all candidates tied at the largest ratio, in table order.
    int best = 0;
    for (int i = 1; i < n3; ++i)
        if (compare_ratio(list[i].c, list[best].c) > 0) best = i;
    Cand s4[TDI8_NUM_CONFIGS];
    int n4 = 0;
    for (int i = 0; i < n3; ++i)
        if (compare_ratio(list[i].c, list[best].c) == 0) s4[n4++] = list[i];
    count[3] = n4;

    // Step 5.
    int64_t fewest = -1;
    for (int i = 0; i < n4; ++i) {
        const int64_t rounds = cdiv(thread_blocks(s4[i].c, M, N), static_cast<int64_t>(hw.num_cu) * s4[i].bpc);
        if (fewest < 0 || rounds < fewest) fewest = rounds;
    }
    int pick = -1;
    for (int i = 0; i < n4; ++i) {
        const int64_t rounds = cdiv(thread_blocks(s4[i].c, M, N), static_cast<int64_t>(hw.num_cu) * s4[i].bpc);
        if (rounds == fewest) {
            ++count[4];
            if (pick < 0) pick = s4[i].c.id;
        }
    }
    if (out) {
        out->id = pick;
        out->route = route;
        for (int i = 0; i < 5; ++i) out->survivors[i] = count[i];
    }
    return pick;
}

int split_k_for(const StaticCfg &c, int M, int N, int K, int num_cu) {
    if (c.family != 0 || M <= 0 || N <= 0 || K <= 0 || K % 16 != 0) return 1;
    const int64_t tiles = static_cast<int64_t>((M + c.bm - 1) / c.bm) * ((N + c.bn - 1) / c.bn);
    int s = 1;
    while (tiles * 2 * s <= num_cu && K / (2 * s) >= 8 * c.bk) s *= 2;
    return s;
}

int predicated_fill(int id, int M, int N, int num_cu) {
    const StaticCfg c = static_cfg(id);
    auto tiles = [&](const StaticCfg &x) { return cdiv(M, x.bm) * cdiv(N, x.bn); };
    if (c.family != 0 || tiles(c) >= num_cu) return id;
    int best = id;
    int64_t best_t = tiles(c);
    for (int j = 0; j < TDI8_NUM_CONFIGS; ++j) {
        const StaticCfg x = static_cfg(j);
        if (x.family != 0 || x.mt != 1 || x.nt != 1 || x.excluded) continue;
        const int64_t t = tiles(x);
        if (t > num_cu) continue;
        if (t > best_t || (t == best_t && best != id && x.bk > static_cfg(best).bk)) {
            best = j;
            best_t = t;
        }
    }
    return best;
}

}  // namespace tdi8
