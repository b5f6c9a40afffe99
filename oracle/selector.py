"""Tile-configuration selection of patent application CN114238853A, in plain Python.

TEST INFRASTRUCTURE (see the package docstring): the product's C++ selector is
checked against this function; neither imports the other.

Source: "一种矩阵乘分片配置选择方法及系统" (method and system for selecting a
matrix-multiply tiling configuration), claims 1 to 7.  Claim 1 gives five
steps; claims 2-6 refine steps 2-5, but their formulas were images and are
missing from the text, so the readings below fill them in.  Each is listed in
the design notes.

A configuration (one compiled kernel) is described by:
  family          'general' or 'skinny'
  mfma_m, mfma_n  M and N extent of one matrix-core instruction tile
  waves_m, waves_n  waves of the thread block along M and N
  m_tiles, n_tiles  per-wave repeats along M and N (the claims' data reuse counts)
  block_k         K extent of one K-tile (the claims' block_k_threads)
  threads         threads per block
  blocks_per_cu   blocks of this kernel resident on one compute unit at once
                  (claim 6's block_per_cu; on the device it comes from the
                  runtime occupancy query, which applies the register, LDS and
                  wave-slot limits)
Derived: block_m_threads = waves_m * mfma_m, block_n_threads = waves_n * mfma_n,
the block tile BM = block_m_threads * m_tiles and BN = block_n_threads * n_tiles.

Hardware description: num_cu, max_threads_per_block, min_active_threads
(claim 3's threshold), skinny_max_m (the largest M, or N, sent to the skinny family).

Readings:
  claim 2 (TCU case): block_m_threads and block_n_threads are multiples of the
      instruction's M and N extents, each at least the smallest instruction
      extent (16), and the block has at most max_threads_per_block threads.
  claim 3: a configuration survives step 2 if blocks_per_cu * threads, the
      register-limited number of active threads on a compute unit, is at least
      min_active_threads (one wave per SIMD: 4 * 64 on CDNA4), and if its
      data-reuse scheme was not excluded by the claim's second alternative, a
      performance test over many product sizes (an input here: Cfg.excluded).
  claim 4: min_theory_block_num = num_cu * blocks_per_cu and
      Thread_Blocks = ceil(m / BM) * ceil(n / BN).  A configuration survives if
      Thread_Blocks >= min_theory_block_num; if none does, every step-2
      survivor is replaced by its reuse-1 sibling (same thread split and
      block_k, m_tiles = n_tiles = 1) and all are kept.
  skinny route (CDNA4 addition): after that fallback, when m <= skinny_max_m,
      the candidates are instead the skinny family with the smallest block
      height BM >= m (else, when n <= skinny_max_m, the smallest block width
      BN >= n: a skinny block streams the large operand once whichever side
      is small); those reaching Thread_Blocks >= num_cu are kept (all if
      none) and of these the smallest block width BN (block height BM on
      the n route), then steps 4 and 5 as below.
  claim 5: the compute-to-memory ratio of a BM x BN tile over a K-tile of
      depth BK is BM*BN*BK / (BM*BK + BK*BN) = BM*BN / (BM + BN) (the B tile's
      width is read with n_tiles).  Step 4 keeps every configuration tied at
      the maximum, compared exactly by cross-multiplication.
  claim 6: Launch_kernel_times = ceil(Thread_Blocks / (num_cu * blocks_per_cu)),
      the number of rounds of resident blocks.  Step 5 keeps the minimum.
      block_per_cu (block_per_cu() below) is the smaller of the claim's two
      quotients: the register quotient, registers a thread may hold over the
      registers it uses, and the shared-memory quotient, the shared memory of
      a compute unit over what one block uses.  On CDNA4 a lane may hold 512
      vector registers (both register files together), allocated in granules
      of 8, so the register quotient counts waves per SIMD (at most the
      SIMD's 8 wave slots); a compute unit has 4 SIMDs, so it holds
      floor(4 * waves per SIMD / waves per block) blocks by registers, and
      floor(160 KiB / LDS per block) by LDS.
  Remaining ties: first in table order.

Rules of the CDNA4 re-derivation that are not steps of the claims (the pages
print no selector output, so against the pages these are PARITY UNPINNED; the
tests pin them only by worked examples of the rules themselves):
  * no_overhang: the step-1 filter on block tiles larger than the problem;
  * the skinny route after claim 4's fallback (m or n <= skinny_max_m);
  * split_k: the K split after the five steps (the contest write-up's Split K
    paragraph gives the atomics, not the slice count), including its measured
    minimum of eight K tiles per slice.
The steps of the claims and claim 6's block_per_cu are pinned: the worked
examples of the claims' steps, and block_per_cu against the device's runtime
occupancy query for every compiled configuration (a GPU test).
"""
from __future__ import annotations

from dataclasses import dataclass, field


def ceil_div(a: int, b: int) -> int:
    return -(-a // b)


@dataclass(frozen=True)
class Hw:
    num_cu: int = 256
    max_threads_per_block: int = 1024
    min_active_threads: int = 256
    skinny_max_m: int = 32


@dataclass(frozen=True)
class CuLimits:
    """Per-compute-unit limits that claim 6's quotients divide (CDNA4 values)."""
    simds: int = 4                 # SIMDs per compute unit
    regs_per_lane: int = 512       # vector registers a lane may hold, both files together
    reg_granule: int = 8           # allocation granule of vector registers
    wave_slots: int = 8            # waves one SIMD holds at once
    lds_bytes: int = 160 * 1024    # LDS (shared memory) of one compute unit
    wave_size: int = 64


def block_per_cu(vgprs: int, agprs: int, lds_per_block: int, threads: int, lim: CuLimits = CuLimits()) -> int:
    """Claim 6: blocks resident on one compute unit, the minimum of the
    register quotient and the shared-memory quotient.  vgprs + agprs are the
    vector registers a lane of the kernel uses (architectural, rounded to a
    multiple of 4 when accumulation registers follow, then accumulation)."""
    used = vgprs + agprs
    alloc = ceil_div(used, lim.reg_granule) * lim.reg_granule
    waves_per_simd = lim.wave_slots if alloc == 0 else min(lim.wave_slots, lim.regs_per_lane // alloc)
    waves_per_block = ceil_div(threads, lim.wave_size)
    by_regs = lim.simds * waves_per_simd // waves_per_block
    by_lds = lim.lds_bytes // lds_per_block if lds_per_block > 0 else by_regs
    return min(by_regs, by_lds)


@dataclass(frozen=True)
class Cfg:
    id: int
    family: str
    mfma_m: int
    mfma_n: int
    waves_m: int
    waves_n: int
    m_tiles: int
    n_tiles: int
    block_k: int
    threads: int
    blocks_per_cu: int
    stages: int = 1   # pipeline depth of the compiled kernel; not used by the selection
    excluded: bool = False  # reuse scheme excluded by claim 3's performance test

    @property
    def block_m_threads(self) -> int:
        return self.waves_m * self.mfma_m

    @property
    def block_n_threads(self) -> int:
        return self.waves_n * self.mfma_n

    @property
    def BM(self) -> int:
        return self.block_m_threads * self.m_tiles

    @property
    def BN(self) -> int:
        return self.block_n_threads * self.n_tiles


@dataclass
class Result:
    id: int
    route: int                      # 0 general, 1 reuse-1 fallback, 2 skinny
    trace: dict = field(default_factory=dict)


def thread_blocks(c: Cfg, m: int, n: int) -> int:
    return ceil_div(m, c.BM) * ceil_div(n, c.BN)


def launch_times(c: Cfg, m: int, n: int, hw: Hw) -> int:
    return ceil_div(thread_blocks(c, m, n), hw.num_cu * c.blocks_per_cu)


def ratio_better(a: Cfg, b: Cfg) -> int:
    """+1 if a's BM*BN/(BM+BN) is larger than b's, 0 if equal, -1 if smaller."""
    lhs = a.BM * a.BN * (b.BM + b.BN)
    rhs = b.BM * b.BN * (a.BM + a.BN)
    return (lhs > rhs) - (lhs < rhs)


def step2_ok(c: Cfg, hw: Hw) -> bool:
    split_ok = (c.block_m_threads % c.mfma_m == 0 and c.block_n_threads % c.mfma_n == 0
                and c.block_m_threads >= 16 and c.block_n_threads >= 16
                and c.threads <= hw.max_threads_per_block)
    return (not c.excluded and split_ok and c.blocks_per_cu >= 1
            and c.blocks_per_cu * c.threads >= hw.min_active_threads)


def reuse1_sibling(c: Cfg, table: list[Cfg]) -> Cfg | None:
    for d in table:
        if (d.family == c.family and d.mfma_m == c.mfma_m and d.mfma_n == c.mfma_n
                and d.waves_m == c.waves_m and d.waves_n == c.waves_n
                and d.block_k == c.block_k and d.m_tiles == 1 and d.n_tiles == 1):
            return d
    return None


def _steps_4_5(cands: list[Cfg], m: int, n: int, hw: Hw, trace: dict) -> Cfg:
    best = cands[0]
    for c in cands[1:]:
        if ratio_better(c, best) > 0:
            best = c
    s4 = [c for c in cands if ratio_better(c, best) == 0]
    trace["step4"] = [c.id for c in s4]
    rounds = min(launch_times(c, m, n, hw) for c in s4)
    s5 = [c for c in s4 if launch_times(c, m, n, hw) == rounds]
    trace["step5"] = [c.id for c in s5]
    return s5[0]


def split_k(c: Cfg, m: int, n: int, k: int, num_cu: int) -> int:
    """K slices for configuration c when its unpredicated form runs (K a
    multiple of 16 bytes).  CDNA4 RULE, NOT A STEP OF THE CLAIMS (parity
    unpinned against the pages): an addition after the five steps, from the
    contest write-up's "Split K" paragraph (partial sums over K slices added
    with integer atomics).  Reading: the slice count s is a power of two, the
    largest with tiles * s <= num_cu (tiles counting the partial ones at the
    ends of M and N) and K / s at least eight K tiles (slices are whole 16-byte
    chunks and need not be whole K tiles); the skinny family never splits."""
    bk = c.block_k
    if c.family != "general" or k % 16 or min(m, n, k) <= 0:
        return 1
    tiles = -(-m // c.BM) * -(-n // c.BN)
    best = 1
    s = 2
    while tiles * s <= num_cu and k // s >= 8 * bk:
        best = s
        s *= 2
    return best


def predicated_fill(c: Cfg, m: int, n: int, num_cu: int, table: list[Cfg]) -> Cfg:
    """Configuration that runs a selected general configuration c when the
    call takes the predicated form with column-major B (operands that the
    16-byte DMA loads cannot move).  CDNA4 RULE, NOT A STEP OF THE CLAIMS
    (parity unpinned against the pages): the selection counts on split_k to
    fill the compute units when its tiles are few, and the predicated
    kernels cannot split K.  Reading: when c's tiles (partial ones at the
    ends of M and N counted) are fewer than num_cu, take among the reuse-1
    general configurations (m_tiles = n_tiles = 1) with at most num_cu tiles
    the one with the most tiles, ties to the deeper K tile, then table
    order; c itself if none has more tiles than c."""
    def tiles(x: Cfg) -> int:
        return -(-m // x.BM) * -(-n // x.BN)
    if c.family != "general" or tiles(c) >= num_cu:
        return c
    best = c
    for x in table:
        if x.family != "general" or x.m_tiles != 1 or x.n_tiles != 1 or x.excluded:
            continue
        t = tiles(x)
        if t > num_cu:
            continue
        if t > tiles(best) or (t == tiles(best) and best is not c and x.block_k > best.block_k):
            best = x
    return best


def no_overhang(cands: list[Cfg], m: int, n: int, table: list[Cfg]) -> list[Cfg]:
    """CDNA4 RULE, NOT A STEP OF THE CLAIMS (parity unpinned against the
    pages), added to step 1: keep the configurations whose block tile is
    no taller than max(m, smallest block height of the general family) and
    no wider than max(n, smallest width); all of them if none is."""
    gen = [c for c in table if c.family == "general"]
    hmin = min(c.BM for c in gen)
    wmin = min(c.BN for c in gen)
    fit = [c for c in cands if c.BM <= max(m, hmin) and c.BN <= max(n, wmin)]
    return fit if fit else list(cands)


def select(m: int, n: int, k: int, hw: Hw, table: list[Cfg]) -> Result:
    """Pick a configuration id for an m x k times k x n product."""
    trace: dict = {}
    general = no_overhang([c for c in table if c.family == "general"], m, n, table)
    trace["step1"] = [c.id for c in general]
    s2 = [c for c in general if step2_ok(c, hw)]
    trace["step2"] = [c.id for c in s2]
    if not s2:
        raise ValueError("no configuration survives step 2")
    s3 = [c for c in s2 if thread_blocks(c, m, n) >= hw.num_cu * c.blocks_per_cu]
    route = 0
    if not s3:
        route = 1
        seen, s3 = set(), []
        for c in s2:
            d = reuse1_sibling(c, table)
            if d is not None and d.id not in seen and step2_ok(d, hw):
                seen.add(d.id)
                s3.append(d)
        s3 = no_overhang(sorted(s3, key=lambda c: c.id), m, n, table)
        if m <= hw.skinny_max_m or n <= hw.skinny_max_m:
            # CDNA4 RULE, NOT A STEP OF THE CLAIMS (parity unpinned against the
            # pages): the skinny route.  A small m picks by block height, else
            # a small n by block width
            ext = (lambda c: c.BM) if m <= hw.skinny_max_m else (lambda c: c.BN)
            small = m if m <= hw.skinny_max_m else n
            skinny = [c for c in table if c.family == "skinny" and ext(c) >= small and step2_ok(c, hw)]
            if skinny:
                e = min(ext(c) for c in skinny)
                skinny = [c for c in skinny if ext(c) == e]
                route = 2
                fill = [c for c in skinny if thread_blocks(c, m, n) >= hw.num_cu]
                s3 = fill if fill else skinny
                # of those, the smallest extent along the other dimension
                other = (lambda c: c.BN) if m <= hw.skinny_max_m else (lambda c: c.BM)
                least = min(other(c) for c in s3)
                s3 = [c for c in s3 if other(c) == least]
    trace["step3"] = [c.id for c in s3]
    trace["route"] = route
    pick = _steps_4_5(s3, m, n, hw, trace)
    return Result(pick.id, route, trace)
