"""Pins for the Python reading of the patent's tile-configuration selector.

The pages print no selector output, so against the pages this is "parity
unpinned".  It is pinned instead by worked examples: each expected id below
was derived by hand from the claims' rules on a small fake table, with the
arithmetic written next to it."""
import pytest

from oracle.selector import Cfg, Hw, select, thread_blocks, launch_times, ratio_better


def table(bpc4=2):
    g = "general"
    s = "skinny"
    return [
        Cfg(0, g, 32, 32, 2, 2, 4, 4, 128, 256, 1),   # 256 x 256
        Cfg(1, g, 32, 32, 2, 2, 2, 2, 128, 256, 2),   # 128 x 128
        Cfg(2, g, 32, 32, 2, 2, 1, 1, 128, 256, 4),   # 64 x 64, reuse-1 sibling of 0, 1, 3
        Cfg(3, g, 32, 32, 2, 2, 2, 1, 128, 256, 2),   # 128 x 64
        Cfg(4, g, 16, 16, 2, 2, 4, 4, 128, 256, bpc4),  # 128 x 128 with 16x16 tiles
        Cfg(5, g, 16, 16, 2, 2, 1, 1, 128, 256, 8),   # 32 x 32, reuse-1 sibling of 4
        Cfg(6, s, 16, 16, 1, 1, 1, 1, 64, 512, 2),    # skinny 16 x 16
        Cfg(7, s, 16, 16, 1, 1, 1, 2, 64, 512, 2),    # skinny 16 x 32
        Cfg(8, s, 16, 16, 1, 1, 2, 1, 64, 512, 2),    # skinny 32 x 16
    ]


HW = Hw(num_cu=256, max_threads_per_block=1024, min_active_threads=256, skinny_max_m=32)


def test_derived_quantities():
    t = table()
    assert (t[0].BM, t[0].BN, t[3].BM, t[3].BN, t[8].BM, t[8].BN) == (256, 256, 128, 64, 32, 16)
    assert thread_blocks(t[0], 4096, 4096) == 256
    assert thread_blocks(t[3], 1000, 3000) == 8 * 47
    assert launch_times(t[0], 16384, 16384, HW) == 16
    assert ratio_better(t[0], t[1]) == 1 and ratio_better(t[1], t[4]) == 0 and ratio_better(t[3], t[1]) == -1


@pytest.mark.parametrize("m,n,want_id,want_route", [
    # 4096^2: every config fills (id0 256 >= 256*1, id1 1024 >= 512, ...); max ratio 256*256/512 = 128 -> id0
    (4096, 4096, 0, 0),
    # 16384^2: id0 has 4096 blocks, still the max ratio -> id0 (16 rounds)
    (16384, 16384, 0, 0),
    # 1000 x 3000: id0 48 < 256, id1 192 < 512, id2 752 < 1024, id3 376 < 512, id4 192 < 512,
    # id5 32*94 = 3008 >= 2048 -> only id5 survives step 3
    (1000, 3000, 5, 0),
    # 256^2: nothing fills (id5 64 < 2048) -> reuse-1 siblings {2, 5}; ratio 32 > 16 -> id2, fallback
    (256, 256, 2, 1),
    # 16 x 4096: fallback, m <= 32 -> skinny with BM = 16: id6 has 256 blocks >= 256, id7 128 < 256 -> id6
    (16, 4096, 6, 2),
    # 16 x 8192: id6 512 and id7 256 both fill; the smallest block width -> id6
    (16, 8192, 6, 2),
    # 17 x 4096: smallest skinny BM >= 17 is 32 -> id8 (256 blocks)
    (17, 4096, 8, 2),
    # 33 x 4096: step 1 keeps block heights <= max(33, 32) = 33, i.e. only id5 (32 x 32);
    # 2 * 128 = 256 < 8 * 256 blocks -> fallback; id5 is its own reuse-1 sibling; too tall
    # for the skinny family -> id5
    (33, 4096, 5, 1),
    # 1 x 1: fallback then skinny; nothing fills, keep {6, 7}; the smallest block width -> id6
    (1, 1, 6, 2),
    # 4096 x 16: M is large, N = 16 small: skinny by block width: smallest BN >= 16 is
    # 16 (id6 16 x 16, id8 32 x 16); id6 256 x 1 = 256 blocks, id8 128 < 256 -> id6
    (4096, 16, 6, 2),
    # 8192 x 16: id6 512 and id8 256 both fill; the smallest block height -> id6
    (8192, 16, 6, 2),
    # 4096 x 17: smallest BN >= 17 is 32 -> id7 (16 x 32, 256 blocks)
    (4096, 17, 7, 2),
    # 4096 x 33: no skinny width reaches 33 and M > 32: the fallback's pick stands;
    # step 1 keeps widths <= max(33, 32): id5 only -> id5
    (4096, 33, 5, 1),
])
def test_worked_examples(m, n, want_id, want_route):
    r = select(m, n, 4096, HW, table())
    assert (r.id, r.route) == (want_id, want_route), r.trace


def test_claim3_register_filter_and_step5_rounds():
    hw = Hw(num_cu=256, max_threads_per_block=1024, min_active_threads=512, skinny_max_m=32)
    # id0 has 1 * 256 = 256 < 512 active threads: dropped at step 2.
    # 4096^2: best ratio 64 shared by id1 and id4; rounds ceil(1024 / 512) = 2 for both -> table order, id1
    r = select(4096, 4096, 4096, hw, table())
    assert 0 not in r.trace["step2"] and r.id == 1 and r.trace["step4"] == [1, 4]
    # with id4 at 4 blocks per CU its rounds drop to ceil(1024 / 1024) = 1 -> id4
    r = select(4096, 4096, 4096, hw, table(bpc4=4))
    assert r.id == 4 and r.trace["step5"] == [4]


def test_other_hardware():
    # 304 compute units: id0 has 256 < 304 blocks at 4096^2 -> out; id1 and id4 tie on ratio 64
    # and on rounds ceil(1024 / 608) = 2 -> id1
    r = select(4096, 4096, 4096, Hw(num_cu=304), table())
    assert r.id == 1 and r.route == 0
    # 256-thread blocks only: the 512-thread skinny kernels are excluded, so 16 x 4096 stays
    # on the reuse-1 fallback; step 1 kept only id5 (block height 32 <= max(16, 32)) -> id5
    r = select(16, 4096, 4096, Hw(max_threads_per_block=256), table())
    assert (r.id, r.route) == (5, 1)


def test_no_overhang_step1():
    """The CDNA4 addition to step 1, worked by hand on the fake table
    (smallest block height and width 32)."""
    # m = 4096, n = 64: widths <= 64 survive: id2 (64 x 64), id3 (128 x 64), id5 (32 x 32);
    # id3: 32 * 1 = 32 blocks < 2 * 256, id2 64 < 4 * 256, id5 256 < 8 * 256 -> fallback;
    # siblings {2, 5} (of 2, 3 and 5), both fit; ratio 32 > 16 -> id2
    r = select(4096, 64, 4096, HW, table())
    assert r.trace["step1"] == [2, 3, 5] and (r.id, r.route) == (2, 1)
    # m = 100, n = 100: heights and widths <= 100: id2 and id5 -> fallback -> id2
    r = select(100, 100, 4096, HW, table())
    assert r.trace["step1"] == [2, 5] and r.id == 2
    # m = 8, n = 8: nothing is within max(8, 32) = 32 but id5 -> id5 survives step 1
    r = select(8, 8, 4096, Hw(skinny_max_m=0), table())
    assert r.trace["step1"] == [5] and (r.id, r.route) == (5, 1)


def test_deterministic_and_k_independent():
    a = [select(m, n, 64, HW, table()).id for m in (1, 16, 100, 4096) for n in (1, 300, 4096)]
    b = [select(m, n, 8192, HW, table()).id for m in (1, 16, 100, 4096) for n in (1, 300, 4096)]
    assert a == b


def test_split_k_worked_examples():
    """The K-split rule (a CDNA4 addition after the five steps), worked by hand:
    slices double while tiles * slices <= #CU (partial tiles counted) and K /
    slices keeps at least eight K tiles; K must be whole 16-byte chunks."""
    from oracle.selector import split_k
    g64x128 = Cfg(10, "general", 32, 32, 2, 4, 1, 1, 128, 512, 3)       # 64 x 128, BK 128
    g256 = Cfg(11, "general", 32, 32, 2, 4, 4, 2, 128, 512, 1)          # 256 x 256
    sk = Cfg(12, "skinny", 16, 16, 1, 1, 1, 1, 2048, 1024, 1)
    assert (g64x128.BM, g64x128.BN, g256.BM, g256.BN) == (64, 128, 256, 256)
    # 256x256x32768: 4*2 = 8 tiles; 8*32 = 256 <= 256 and 32768/32 = 1024 >= 8*128 -> 32
    assert split_k(g64x128, 256, 256, 32768, 256) == 32
    # 1024x1024x8192: 16*8 = 128 tiles; 2 slices fill 256 exactly -> 2
    assert split_k(g64x128, 1024, 1024, 8192, 256) == 2
    # 4096^3 with 256x256: 256 tiles, no room -> 1
    assert split_k(g256, 4096, 4096, 4096, 256) == 1
    # K = 2048: two slices of 1024 = 8 tiles of 128; four slices would be 512 -> 2
    assert split_k(g64x128, 256, 256, 2048, 256) == 2
    # K = 1536: two slices of 768 < 1024 -> 1
    assert split_k(g64x128, 256, 256, 1536, 256) == 1
    # K = 3072: 1536 >= 1024 -> 2; 768 < 1024 -> stop
    assert split_k(g64x128, 256, 256, 3072, 256) == 2
    # K = 2176 = 17 K tiles: 1088 >= 1024 -> 2 (slices of 8.5 K tiles); 544 < 1024 -> stop
    assert split_k(g64x128, 256, 256, 2176, 256) == 2
    # K = 2064 = 129 chunks of 16: 1032 >= 1024 -> 2 (slices of 65 and 64 chunks)
    assert split_k(g64x128, 64, 128, 2064, 256) == 2
    # tile-ragged M = 100: 2 x 2 = 4 tiles (one partial row of tiles); 4 * 32 = 128 <= 256
    # and 32768 / 32 = 1024 >= 1024 -> 32; 32768 / 64 = 512 < 1024 -> stop
    assert split_k(g64x128, 100, 256, 32768, 256) == 32
    # 500 x 500: 8 x 4 = 32 tiles; 32 * 8 = 256 and 16384 / 8 = 2048 >= 1024 -> 8
    assert split_k(g64x128, 500, 500, 16384, 256) == 8
    # K not whole 16-byte chunks, the skinny family: never split
    assert split_k(g64x128, 256, 256, 32776, 256) == 1
    assert split_k(sk, 16, 4096, 65536, 256) == 1
    # 120 compute units, 8 tiles: 16 * 8 = 128 > 120 -> 8
    assert split_k(g64x128, 256, 256, 32768, 120) == 8


def test_predicated_fill_worked_examples():
    """The predicated-form fill rule (a CDNA4 addition after the five steps),
    worked by hand: when the selected tiles number fewer than the compute
    units, the reuse-1 general configuration with the most tiles, at most
    one per compute unit, runs instead; ties to the deeper K tile, then
    table order; the selected one stays if no such configuration has more
    tiles.  Tiles count the partial ones at the ends of M and N."""
    from oracle.selector import predicated_fill
    g = "general"
    g64x128 = Cfg(7, g, 32, 32, 2, 4, 1, 1, 128, 512, 2)    # 64 x 128, BK 128
    g128x64 = Cfg(9, g, 32, 32, 4, 2, 1, 1, 128, 512, 2)    # 128 x 64, BK 128
    g64x64a = Cfg(5, g, 32, 32, 2, 2, 1, 1, 64, 256, 4)     # 64 x 64, BK 64
    g64x64b = Cfg(11, g, 32, 32, 2, 2, 1, 1, 128, 256, 4)   # 64 x 64, BK 128
    g256 = Cfg(0, g, 32, 32, 2, 4, 4, 2, 128, 512, 1)       # 256 x 256
    sk = Cfg(12, "skinny", 16, 16, 1, 1, 1, 1, 2048, 1024, 1)
    tab = [g256, g64x64a, g64x128, g128x64, g64x64b, sk]
    # 1000 x 1000: 64 x 128 -> 16 * 8 = 128 tiles < 256; 64 x 64 -> 16 * 16 = 256 (both BK);
    # 128 x 64 -> 8 * 16 = 128: the 64 x 64 pair ties at 256, the deeper K tile wins
    assert predicated_fill(g64x128, 1000, 1000, 256, tab) is g64x64b
    # 512 x 512: 8 * 4 = 32 tiles; 64 x 64 -> 64
    assert predicated_fill(g64x128, 512, 512, 256, tab) is g64x64b
    # 333 x 777: 6 * 7 = 42 tiles; 64 x 64 -> 6 * 13 = 78; 128 x 64 -> 3 * 13 = 39
    assert predicated_fill(g64x128, 333, 777, 256, tab) is g64x64b
    # 1000 x 3000: 16 * 24 = 384 >= 256 tiles: the selected configuration stays
    assert predicated_fill(g64x128, 1000, 3000, 256, tab) is g64x128
    # 1000 x 2000: 16 * 16 = 256: stays (no idle compute unit)
    assert predicated_fill(g64x128, 1000, 2000, 256, tab) is g64x128
    # 1500 x 1500 with 256 x 256 selected: 6 * 6 = 36 tiles; 64 x 64 -> 24 * 24 = 576 > 256 and
    # 64 x 128 -> 24 * 12 = 288 > 256 are too many; 128 x 64 -> 12 * 24 = 288 too: none fits, it stays
    assert predicated_fill(g256, 1500, 1500, 256, tab) is g256
    # 900 x 900 with 256 x 256 selected: 4 * 4 = 16; 64 x 64 -> 15 * 15 = 225 <= 256
    assert predicated_fill(g256, 900, 900, 256, tab) is g64x64b
    # 120 compute units: 512 x 512 -> 64 x 64 gives 64 tiles <= 120
    assert predicated_fill(g64x128, 512, 512, 120, tab) is g64x64b
    # a tie in tiles with the selected one is no gain: 128 x 64 at 1000 x 1000 (128 tiles) keeps 64 x 128
    assert predicated_fill(g64x128, 1000, 1000, 256, [g64x128, g128x64]) is g64x128
    # the skinny family is never moved
    assert predicated_fill(sk, 16, 100, 256, tab) is sk


def test_claim3_excluded_reuse_scheme():
    """Claim 3's second alternative drops a reuse scheme at step 2.  Scheme
    4 x 4 of the fake table is id0 (256 x 256) and id4 (128 x 128, 16x16
    tiles).  4096^2 without them: id1 (1024 >= 512 blocks), id2, id3 and id5
    fill; the largest ratio 128*128/256 = 64 belongs to id1 alone -> id1."""
    import dataclasses
    tab = [dataclasses.replace(c, excluded=c.family == "general" and (c.m_tiles, c.n_tiles) == (4, 4))
           for c in table()]
    r = select(4096, 4096, 4096, HW, tab)
    assert r.trace["step2"] == [1, 2, 3, 5] and r.id == 1 and r.route == 0
    # 256^2 falls back as before: the siblings {2, 5} are reuse 1 and stay -> id2
    r = select(256, 256, 4096, HW, tab)
    assert (r.id, r.route) == (2, 1)


def test_reuse_scheme_test_rule():
    """The performance test's rule, on hand-made timings (µs): relative speed
    = fastest time on the shape / the scheme's fastest time there."""
    import importlib.util, os
    spec = importlib.util.spec_from_file_location(
        "bench_for_test", os.path.join(os.path.dirname(os.path.dirname(__file__)), "bench.py"))
    bench = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(bench)

    class C:
        def __init__(self, id, fam, mt, nt):
            self.id, self.family, self.m_tiles, self.n_tiles = id, fam, mt, nt

    tab = [C(0, 0, 4, 2), C(1, 0, 4, 4), C(2, 0, 1, 1), C(3, 0, 2, 2), C(4, 0, 4, 4), C(5, 1, 1, 2)]
    times = {
        "a": {0: 10.0, 1: 12.5, 2: 20.0, 3: 11.0, 4: 30.0},   # best 10: scheme 4x4 -> 10/12.5 = 0.8
        "b": {0: 50.0, 1: 80.0, 2: 40.0, 3: 100.0, 4: 70.0},  # best 40: 4x4 -> 40/70 = 0.571, 2x2 -> 0.4
        "c": {2: 9.0, 5: 10.0},                                # only the 1x1 and skinny 1x2 timed
    }
    rows = {r[0]: r for r in bench.reuse_pruning(times, tab, theta=0.85)}
    # 4x4: 0.8 and 0.571, below 0.85 on both of its tests -> excluded
    key, ids, ntest, lo, hi, excl = rows[(0, 4, 4)]
    assert ids == [1, 4] and ntest == 2 and abs(lo - 40 / 70) < 1e-12 and abs(hi - 0.8) < 1e-12 and excl
    # 2x2: 10/11 = 0.909 on "a" -> kept though 0.4 on "b"
    assert rows[(0, 2, 2)][5] is False and abs(rows[(0, 2, 2)][4] - 10 / 11) < 1e-12
    # 1x1: 0.5, 1.0 and 1.0; reuse 1 is kept in any case
    assert rows[(0, 1, 1)][5] is False
    # skinny 1x2: 9/10 = 0.9 on its one test -> kept; at threshold 0.95 -> excluded
    assert rows[(1, 1, 2)][2] == 1 and rows[(1, 1, 2)][5] is False
    assert {r[0]: r for r in bench.reuse_pruning(times, tab, theta=0.95)}[(1, 1, 2)][5] is True
    # 4x2: the fastest on "a" -> kept
    assert rows[(0, 4, 2)][5] is False
