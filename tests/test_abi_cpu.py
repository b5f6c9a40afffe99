"""Host-side checks of the C-ABI library (no GPU): it loads, exports every
function include/tdi8.h declares, validates arguments, and its selection
agrees with the oracle's reading of the patent on described hardware."""
import ctypes
import os
import re

import pytest

import tiled_dense_int8_amd as t
from oracle.selector import Cfg, CuLimits, Hw, block_per_cu, select

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "tdi8.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))


def test_header_functions_are_exported():
    names = declared_functions()
    assert "gemm_s8s8s32" in names and "select_tile_config" in names and len(names) >= 10
    lib = ctypes.CDLL(t.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(t.EXPORTED) == names


def test_nm_shows_c_linkage():
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", t.LIB_PATH], capture_output=True, text=True).stdout
    syms = {line.split()[-1] for line in out.splitlines() if line.strip()}
    for n in declared_functions():
        assert n in syms, n


def test_status_strings():
    for st in range(0, -7, -1):
        assert t.tdi8_status_string(st) and t.tdi8_status_string(st) != "unknown status"
    assert t.tdi8_status_string(-99) == "unknown status"


A, B, C = 0x10000, 0x20000000, 0x40000000  # fake, well separated addresses; nothing is dereferenced


@pytest.mark.parametrize("bcm", [0, 1])
def test_validation(bcm):
    v = t.tdi8_validate
    ldb = 64 if bcm else 32
    assert v(bcm, 16, 32, 64, A, 64, B, ldb, C, 32) == t.OK
    assert v(bcm, -1, 32, 64, A, 64, B, ldb, C, 32) == t.ERR_INVALID_VALUE
    assert v(bcm, 16, -1, 64, A, 64, B, ldb, C, 32) == t.ERR_INVALID_VALUE
    assert v(bcm, 16, 32, -5, A, 64, B, ldb, C, 32) == t.ERR_INVALID_VALUE
    assert v(bcm, 16, 32, 64, A, 63, B, ldb, C, 32) == t.ERR_INVALID_VALUE       # lda < K
    assert v(bcm, 16, 32, 64, A, 64, B, ldb - 1, C, 32) == t.ERR_INVALID_VALUE   # ldb too small
    assert v(bcm, 16, 32, 64, A, 64, B, ldb, C, 31) == t.ERR_INVALID_VALUE       # ldc < N
    assert v(bcm, 16, 32, 64, 0, 64, B, ldb, C, 32) == t.ERR_NULL_POINTER
    assert v(bcm, 16, 32, 64, A, 64, 0, ldb, C, 32) == t.ERR_NULL_POINTER
    assert v(bcm, 16, 32, 64, A, 64, B, ldb, 0, 32) == t.ERR_NULL_POINTER
    # empty problems need no pointers; K == 0 needs only C
    assert v(bcm, 0, 32, 64, 0, 64, 0, ldb, 0, 32) == t.OK
    assert v(bcm, 16, 0, 64, 0, 64, 0, max(ldb, 64), 0, 1) == t.OK
    assert v(bcm, 16, 32, 0, 0, 1, 0, 32, C, 32) == t.OK
    assert v(bcm, 16, 32, 0, 0, 1, 0, 32, 0, 32) == t.ERR_NULL_POINTER
    # C overlapping A or B
    assert v(bcm, 16, 32, 64, A, 64, B, ldb, A + 100, 32) == t.ERR_ALIASING
    assert v(bcm, 16, 32, 64, A, 64, B, ldb, B + 8, 32) == t.ERR_ALIASING
    assert v(bcm, 16, 32, 64, A, 64, B, ldb, A - 4 * (15 * 32 + 32) + 1, 32) == t.ERR_ALIASING
    assert v(bcm, 16, 32, 64, A, 64, B, ldb, A - 4 * (15 * 32 + 32), 32) == t.OK  # ends exactly at A


def test_entry_points_reject_before_any_device_work():
    # invalid arguments are refused on the host, with no device present
    assert t.gemm_s8s8s32(-1, 4, 4, A, 4, B, 4, C, 4, 0) == t.ERR_INVALID_VALUE
    assert t.gemm_s8s8s32_bt(4, 4, 4, A, 4, B, 3, C, 4, 0) == t.ERR_INVALID_VALUE
    assert t.gemm_s8s8s32_with_config(99, 1, 4, 4, 4, A, 4, B, 4, C, 4, 0) == t.ERR_BAD_CONFIG
    assert t.gemm_s8s8s32_with_config(-1, 1, 4, 4, 4, A, 4, B, 4, C, 4, 0) == t.ERR_BAD_CONFIG
    assert t.gemm_s8s8s32(0, 4, 4, 0, 4, 0, 4, 0, 4, 0) == t.OK
    assert t.select_tile_config(-1, 1, 1) == t.ERR_INVALID_VALUE
    # the persistent form: same argument checks, then its own
    p = t.gemm_s8s8s32_persistent
    assert p(0, 1, -1, 4, 4, A, 4, B, 4, C, 4, 0, 0) == t.ERR_INVALID_VALUE
    assert p(0, 1, 4, 4, 4, None, 4, B, 4, C, 4, 0, 0) == t.ERR_NULL_POINTER
    assert p(0, 0, 4, 4, 4, A, 4, B, 4, A + 2, 4, 0, 0) == t.ERR_ALIASING
    assert p(99, 1, 4, 4, 4, A, 4, B, 4, C, 4, 0, 0) == t.ERR_BAD_CONFIG
    assert p(-2, 1, 4, 4, 4, A, 4, B, 4, C, 4, 0, 0) == t.ERR_BAD_CONFIG
    assert p(0, 1, 4, 4, 4, A, 4, B, 4, C, 4, -1, 0) == t.ERR_INVALID_VALUE
    assert p(0, 1, 0, 4, 4, 0, 4, 0, 4, 0, 4, 0, 0) == t.OK


def library_table():
    return [t.tile_config_info(i) for i in range(t.tile_config_count())]


def test_config_table_shape():
    tab = library_table()
    assert [c.id for c in tab] == list(range(len(tab)))
    for c in tab:
        assert c.block_m == c.waves_m * c.mfma_m * c.m_tiles
        assert c.block_n == c.waves_n * c.mfma_n * c.n_tiles
        assert c.threads == 64 * c.waves_m * c.waves_n * c.waves_k
        assert c.mfma_k == (32 if c.mfma_m == 32 else 64)
        if c.family == 1:
            # the skinny family has no fallback of its own: a sibling is optional
            assert c.reuse1_id == -1 or tab[c.reuse1_id].m_tiles == tab[c.reuse1_id].n_tiles == 1
            assert c.lds_bytes <= 160 * 1024
            continue
        sib = tab[c.reuse1_id]
        # the sibling keeps the thread split and K tile; its pipeline depth may differ
        assert (sib.family, sib.mfma_m, sib.waves_m, sib.waves_n, sib.waves_k, sib.block_k,
                sib.m_tiles, sib.n_tiles) == (c.family, c.mfma_m, c.waves_m, c.waves_n, c.waves_k, c.block_k, 1, 1)
        if c.family == 0:
            assert c.lds_bytes == c.stages * (c.block_m + c.block_n) * c.block_k <= 160 * 1024
            assert c.stages >= 2 and (c.block_k // (32 if c.mfma_m == 32 else 64)) % 2 == 0
    assert any(c.family == 1 and c.block_m == 16 for c in tab)
    assert any(c.family == 1 and c.block_m == 32 for c in tab)


def oracle_table(bpc):
    fam = {0: "general", 1: "skinny"}
    return [Cfg(c.id, fam[c.family], c.mfma_m, c.mfma_n, c.waves_m, c.waves_n, c.m_tiles, c.n_tiles,
                c.block_k, c.threads, bpc[c.id], c.stages, bool(c.excluded)) for c in library_table()]


def claim6_bpc(lim=CuLimits()):
    """Resident blocks per CU of every compiled configuration by claim 6's
    quotients (the oracle's block_per_cu) from the registers and LDS the
    build read out of each kernel, on described compute-unit limits."""
    return [block_per_cu(c.vgprs, c.agprs, c.lds_bytes, c.threads, lim) for c in library_table()]


HARDWARE = [
    (Hw(256, 1024, 256, 32), claim6_bpc()),
    (Hw(256, 1024, 256, 32), [1] * 64),
    (Hw(304, 1024, 256, 32), claim6_bpc(CuLimits(lds_bytes=64 * 1024))),
    (Hw(80, 256, 128, 16), claim6_bpc(CuLimits(lds_bytes=64 * 1024, regs_per_lane=256, wave_slots=4))),
    (Hw(256, 1024, 1024, 32), claim6_bpc()),
]


def test_kernel_resources_from_the_build():
    """Register and LDS figures come from the compiled code objects: the
    general kernels' LDS is exactly their stage buffers, every kernel fits
    the 512 registers of a lane, and architectural registers that precede
    accumulation registers are a multiple of 4."""
    for c in library_table():
        assert c.vgprs > 0 and c.sgprs > 0 and c.agprs >= 0
        assert c.vgprs + c.agprs <= 512
        if c.agprs:
            assert c.vgprs % 4 == 0
        assert 0 < c.lds_bytes <= 160 * 1024
    # the 4-wave 256 x 256 tiles hold 16 accumulator tiles of 16 registers per lane
    tab = library_table()
    assert any(c.agprs == 256 for c in tab if c.block_m == c.block_n == 256 and c.threads == 256)


def test_claim6_block_per_cu_worked_examples():
    """Claim 6's quotients worked by hand on CDNA4's limits (512 registers a
    lane in granules of 8, 8 wave slots per SIMD, 4 SIMDs, 160 KiB LDS)."""
    # 216 registers -> 2 waves per SIMD -> 8 waves per CU -> one 8-wave block; LDS 160/128 -> 1
    assert block_per_cu(216, 0, 131072, 512) == 1
    # 56 + 16 = 72 registers -> 7 waves per SIMD -> 28 waves -> 7 four-wave blocks; LDS 160/32 -> 5
    assert block_per_cu(56, 16, 32768, 256) == 5
    # the same without LDS: the register quotient decides
    assert block_per_cu(56, 16, 0, 256) == 7
    # 83 registers allocate 88 -> 5 waves per SIMD -> 20 waves -> two 8-wave blocks
    assert block_per_cu(83, 0, 1024, 512) == 2
    # few registers: the 8 wave slots cap the quotient (32 waves -> two 16-wave blocks)
    assert block_per_cu(38, 0, 1024, 1024) == 2
    # 104 + 256 = 360 registers -> one wave per SIMD -> one 4-wave block
    assert block_per_cu(104, 256, 65536, 256) == 1
    # a kernel too large for the hardware described gets 0
    assert block_per_cu(300, 0, 1024, 512, CuLimits(regs_per_lane=256)) == 0
    assert block_per_cu(64, 0, 200 * 1024, 256) == 0
    # granule: 129 registers allocate 136 -> 3 waves, 128 allocate 128 -> 4
    assert block_per_cu(129, 0, 0, 256) == 3 and block_per_cu(128, 0, 0, 256) == 4


def test_gemm_plan_host_checks():
    """gemm_plan refuses bad arguments with the gemm call's status codes,
    before any device work, and an empty product plans nothing."""
    with pytest.raises(t.TDI8Error) as e:
        t.gemm_plan(-1, 1, -1, 4, 4, A, 4, B, 4, C, 4)
    assert e.value.status == t.ERR_INVALID_VALUE
    with pytest.raises(t.TDI8Error) as e:
        t.gemm_plan(99, 1, 4, 4, 4, A, 4, B, 4, C, 4)
    assert e.value.status == t.ERR_BAD_CONFIG
    with pytest.raises(t.TDI8Error) as e:
        t.gemm_plan(-1, 0, 4, 4, 4, A, 4, B, 4, A + 2, 4)
    assert e.value.status == t.ERR_ALIASING
    p = t.gemm_plan(-1, 1, 0, 4, 4, 0, 4, 0, 4, 0, 4)
    assert (p.form, p.kernels, p.config_id) == (t.FORM_NONE, 0, -1)
    assert t._lib.gemm_plan(-1, 1, 4, 4, 4, A, 4, B, 4, C, 4, None) == t.ERR_NULL_POINTER


def test_int_arguments_beyond_int32_are_refused():
    """ctypes would wrap a Python int past 2**31 - 1 silently (2**32 + 5
    arrives as 5); the binding refuses it before calling the library."""
    for bad in (2 ** 31, 2 ** 32 + 5, -2 ** 31 - 1):
        with pytest.raises(ValueError):
            t.gemm_s8s8s32(bad, 4, 4, A, 4, B, 4, C, 4, 0)
        with pytest.raises(ValueError):
            t.gemm_s8s8s32_bt(4, 4, 4, A, bad, B, 4, C, 4, 0)
        with pytest.raises(ValueError):
            t.gemm_s8s8s32_with_config(0, 1, 4, 4, 4, A, 4, B, 4, C, bad, 0)
        with pytest.raises(ValueError):
            t.select_tile_config(4, bad, 4)
        with pytest.raises(ValueError):
            t.tdi8_validate(1, 4, 4, bad, A, 4, B, 4, C, 4)
        with pytest.raises(ValueError):
            t.conv2d_s8s8s32_nhwc(1, bad, 8, 16, 4, 3, 3, 1, 1, 1, 1, 1, 1, A, B, C, 0)
        with pytest.raises(ValueError):
            t.conv2d_output_extent(bad, 3, 1, 1, 1)
    # the largest int passes through to the library's own checks
    assert t.gemm_s8s8s32(t.INT_MAX, 4, 4, A, 3, B, 4, C, 4, 0) == t.ERR_INVALID_VALUE  # lda < K
SHAPES = [(m, n) for m in (1, 7, 16, 17, 32, 33, 64, 100, 256, 1000, 4096, 16384)
          for n in (1, 16, 100, 256, 3000, 4096, 8192, 16384)]


@pytest.mark.parametrize("hw_index", range(len(HARDWARE)))
def test_selection_matches_oracle_reading(hw_index):
    hw, bpc = HARDWARE[hw_index]
    bpc = list(bpc)[:t.tile_config_count()]
    hwc = t.HwInfo(hw.num_cu, hw.max_threads_per_block, hw.min_active_threads, hw.skinny_max_m)
    table = oracle_table(bpc)
    for m, n in SHAPES:
        try:
            want = select(m, n, 512, hw, table)
        except ValueError:
            with pytest.raises(t.TDI8Error):
                t.select_tile_config_for(m, n, 512, hwc, bpc)
            continue
        got = t.select_tile_config_for(m, n, 512, hwc, bpc)
        assert (got.id, got.route) == (want.id, want.route), (m, n, want.trace)
        assert got.survivors[3] == len(want.trace["step4"]) and got.survivors[4] == len(want.trace["step5"])


def test_mi355x_expectations():
    """With the MI355X description and claim 6's occupancy, the selection
    routes the five workloads as the method intends."""
    hwc = t.HwInfo(256, 1024, 256, 32)
    bpc = claim6_bpc()
    tab = library_table()
    s = t.select_tile_config_for(4096, 4096, 4096, hwc, bpc)
    assert s.route == t.ROUTE_GENERAL and (tab[s.id].block_m, tab[s.id].block_n) == (256, 256)
    s = t.select_tile_config_for(16384, 16384, 8192, hwc, bpc)
    assert s.route == t.ROUTE_GENERAL and (tab[s.id].block_m, tab[s.id].block_n) == (256, 256)
    s = t.select_tile_config_for(16, 4096, 4096, hwc, bpc)
    assert s.route == t.ROUTE_SKINNY and tab[s.id].block_m == 16
    s = t.select_tile_config_for(256, 256, 256, hwc, bpc)
    assert s.route == t.ROUTE_FALLBACK and tab[s.id].m_tiles == tab[s.id].n_tiles == 1
    # a small N routes to the skinny family by block width
    s = t.select_tile_config_for(4096, 16, 4096, hwc, bpc)
    assert s.route == t.ROUTE_SKINNY and tab[s.id].block_n == 16


def test_split_k_matches_oracle_reading():
    """The library's K-split rule against the oracle's restatement, on a grid
    of shapes and compute-unit counts (no device needed)."""
    from oracle.selector import split_k
    tab = oracle_table([1] * t.tile_config_count())
    shapes = [(m, n, k) for m in (64, 128, 256, 1024, 4096, 100) for n in (64, 128, 256, 1024, 3000)
              for k in (128, 256, 512, 768, 1024, 4096, 8192, 32768, 65536, 777)]
    for num_cu in (256, 120, 304, 8):
        for c in tab:
            for (m, n, k) in shapes:
                assert t.tile_config_split_k(c.id, m, n, k, num_cu) == split_k(c, m, n, k, num_cu), (c.id, m, n, k, num_cu)
    assert t.tile_config_split_k(-1, 1, 1, 1, 256) == t.ERR_BAD_CONFIG
    assert t.tile_config_split_k(0, -1, 1, 1, 256) == t.ERR_INVALID_VALUE
    assert t.tile_config_split_k(0, 1, 1, 1, 0) == t.ERR_INVALID_VALUE


def test_conv_validation_and_extent():
    """Host-side checks of the convolution entry (no device needed)."""
    A16 = 1 << 20      # a 16-byte aligned fake address; nothing is dereferenced
    good = (2, 8, 8, 16, 4, 3, 3, 1, 1, 1, 1, 1, 1)
    assert t.conv2d_output_extent(56, 3, 1, 1, 1) == 56
    assert t.conv2d_output_extent(56, 3, 1, 2, 1) == 28
    assert t.conv2d_output_extent(7, 3, 0, 1, 3) == 1
    assert t.conv2d_output_extent(3, 3, 0, 1, 2) == 0
    assert t.conv2d_output_extent(8, 3, -1, 1, 1) == t.ERR_INVALID_VALUE
    assert t.conv2d_output_extent(8, 3, 1, 0, 1) == t.ERR_INVALID_VALUE
    assert t.conv2d_validate(*good, A16, A16 + (1 << 16), A16 + (1 << 17)) == t.OK
    # any channel count and any alignment of x and w (the byte-gather form)
    odd_channels = (2, 8, 8, 3, 4, 3, 3, 1, 1, 1, 1, 1, 1)
    assert t.conv2d_validate(*odd_channels, A16 + 1, A16 + (1 << 16) + 3, A16 + (1 << 17)) == t.OK
    for i, v in [(0, -1), (7, -1), (9, 0), (11, 0), (5, 0)]:
        args = list(good)
        args[i] = v
        assert t.conv2d_validate(*args, A16, A16 + (1 << 16), A16 + (1 << 17)) == t.ERR_INVALID_VALUE, (i, v)
    assert t.conv2d_validate(*good, 0, A16, A16 + (1 << 17)) == t.ERR_NULL_POINTER
    assert t.conv2d_validate(*good, A16, A16 + (1 << 16), 0) == t.ERR_NULL_POINTER
    assert t.conv2d_validate(*good, A16, A16 + (1 << 16), A16 + (1 << 17) + 2) == t.ERR_INVALID_VALUE
    # y overlapping x: 2*8*8*16 bytes of x at A16, y starts inside it
    assert t.conv2d_validate(*good, A16, A16 + (1 << 16), A16 + 64) == t.ERR_ALIASING
    # empty output: nothing to check beyond the sizes
    assert t.conv2d_validate(0, 8, 8, 16, 4, 3, 3, 1, 1, 1, 1, 1, 1, 0, 0, 0) == t.OK
    # entry points reject before any device work
    assert t.conv2d_s8s8s32_nhwc(*good, A16, A16 + (1 << 16), A16 + (1 << 17) + 2, 0) == t.ERR_INVALID_VALUE
    assert t.conv2d_s8s8s32_nhwc_with_config(99, *good, A16, A16 + (1 << 16), A16 + (1 << 17), 0) == t.ERR_BAD_CONFIG


def test_torch_wrappers_refuse_host_tensors_and_bad_arguments():
    """The torch wrappers check their tensors before anything reaches the
    library: host tensors (whose data pointers the kernels would read as
    device addresses), wrong dtypes, mismatched shapes."""
    import torch
    A = torch.zeros((4, 8), dtype=torch.int8)
    B = torch.zeros((8, 4), dtype=torch.int8)
    with pytest.raises(ValueError, match="GPU"):
        t.gemm(A, B, False)
    with pytest.raises(TypeError):
        t.gemm(A.to(torch.int16), B, False)
    with pytest.raises(ValueError, match="inner"):
        t.gemm(A, B[:4], False)
    x = torch.zeros((1, 5, 5, 16), dtype=torch.int8)
    w = torch.zeros((8, 3, 3, 16), dtype=torch.int8)
    with pytest.raises(ValueError, match="GPU"):
        t.conv2d(x, w, (1, 1))
    with pytest.raises(TypeError):
        t.conv2d(x.to(torch.int32), w, (1, 1))
    with pytest.raises(ValueError, match="channel"):
        t.conv2d(x, w[..., :8].contiguous(), (1, 1))
    with pytest.raises(ValueError, match="contiguous"):
        t.conv2d(x.permute(0, 2, 1, 3), w, (1, 1))


def test_ceilings_library_exports_its_header():
    """The calibration library (bench.py --ceilings) loads and exports every
    function its header declares; host-side argument checks need no device."""
    path = os.path.join(os.path.dirname(t.LIB_PATH), "libtdi8_ceilings.so")
    header = os.path.join(os.path.dirname(HEADER), "tdi8_ceilings.h")
    text = re.sub(r"/\*.*?\*/", "", open(header).read(), flags=re.S)
    names = sorted(set(re.findall(r"^\s*int\s+(\w+)\s*\(", text, flags=re.M)))
    assert names == ["tdi8c_dma_read", "tdi8c_empty", "tdi8c_load16", "tdi8c_loop_mix", "tdi8c_mfma_loop",
                     "tdi8c_store_tiles", "tdi8c_stream_read"]
    lib = ctypes.CDLL(path)
    for n in names:
        assert hasattr(lib, n), n
    lib.tdi8c_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    assert lib.tdi8c_stream_read(None, 16, 1, None, None) == -1
    assert lib.tdi8c_stream_read(A, 15, 1, C, None) == -2
    lib.tdi8c_empty.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    assert lib.tdi8c_empty(1, 2048, None) == -2
    lib.tdi8c_dma_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                   ctypes.c_void_p, ctypes.c_void_p]
    assert lib.tdi8c_dma_read(None, 1 << 20, 16, 256, 1, C, None) == -1
    assert lib.tdi8c_dma_read(A, 1 << 20, 8, 256, 1, C, None) == -2     # 128 KiB slabs
    assert lib.tdi8c_dma_read(A, 1 << 20, 16, 100, 1, C, None) == -2    # not whole waves
    lib.tdi8c_loop_mix.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                   ctypes.c_void_p, ctypes.c_void_p]
    assert lib.tdi8c_loop_mix(None, 7, 1, 1, C, C, None) == -1
    assert lib.tdi8c_loop_mix(A, 8, 1, 1, C, C, None) == -2              # no such mode
    lib.tdi8c_store_tiles.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int64, ctypes.c_int,
                                      ctypes.c_void_p]
    assert lib.tdi8c_store_tiles(None, 1, 1, 256, 0, None) == -1
    assert lib.tdi8c_store_tiles(C, 1, 2, 256, 0, None) == -2            # rows shorter than two tiles


def test_stamps_library_exports_the_api_and_its_header():
    """The instrumented build (bench.py --stamps) exports every function of
    tdi8.h and of tdi8_stamps.h; the product library exports no stamp call."""
    path = os.path.join(os.path.dirname(t.LIB_PATH), "libtdi8_stamps.so")
    header = os.path.join(os.path.dirname(HEADER), "tdi8_stamps.h")
    text = re.sub(r"/\*.*?\*/", "", open(header).read(), flags=re.S)
    names = sorted(set(re.findall(r"^\s*int\s+(\w+)\s*\(", text, flags=re.M)))
    assert names == ["tdi8_stamps_set"]
    lib = ctypes.CDLL(path)
    for n in names + declared_functions():
        assert hasattr(lib, n), n
    assert not hasattr(ctypes.CDLL(t.LIB_PATH), "tdi8_stamps_set")
    lib.tdi8_stamps_set.argtypes = [ctypes.c_void_p, ctypes.c_int]
    assert lib.tdi8_stamps_set(None, 4) == t.ERR_INVALID_VALUE
    assert lib.tdi8_stamps_set(None, -1) == t.ERR_INVALID_VALUE
    assert lib.tdi8_stamps_set(None, 0) == t.OK
