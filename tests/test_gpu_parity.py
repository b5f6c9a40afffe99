"""Parity of the HIP path with the CPU oracle, through the C ABI.

Integer work, so the bar is bit-exact equality on every compared element.
Small and ragged shapes are compared in full for every compiled
configuration and both B layouts; the five workload shapes are compared in
full where the oracle finishes in seconds, otherwise on sampled elements
(whole first/last rows and columns plus random positions) together with a
Freivalds product check over the whole of C."""
import numpy as np
import pytest

import synthetic
from helpers import DeviceCase, check_case, note

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import tiled_dense_int8_amd as t
    return t


def table(t):
    return [t.tile_config_info(i) for i in range(t.tile_config_count())]


def shapes_for(c):
    BM, BN, BK = c.block_m, c.block_n, c.block_k
    out = [(BM, BN, BK), (2 * BM, 2 * BN, 2 * BK), (BM + 1, BN - 1, BK + 27), (1, 1, 1), (17, 33, 63),
           (3, 200, 4), (255, 257, 777), (64, 64, 65)]
    if c.family == 0:
        # whole tiles, unsplit, more K tiles than stages: the steady state of
        # the pipelined loop (each iteration refilling the buffer it frees)
        out += [(BM, BN, 8 * BK), (2 * BM, 2 * BN, 6 * BK)]
    if c.family == 1:
        # the last two: unpredicated forms with 8 and 24 column blocks (block renumbering across XCDs)
        out += [(BM, 64, 64), (BM, 128, 256), (BM, 8 * BN, 2 * BK), (2 * BM, 24 * BN, BK)]
    return out


def plan_of(case: DeviceCase, config=-1):
    """The form the library reports for this call (gemm_plan)."""
    import tiled_dense_int8_amd as t
    return t.gemm_plan(config, case.bcm, case.M, case.N, case.K, case.A_ptr, case.lda, case.B_ptr, case.ldb,
                       case.C_ptr, case.ldc)


@pytest.mark.parametrize("bcm", [True, False])
def test_every_config_small_and_ragged(lib, bcm):
    t = lib
    steady = 0
    for c in table(t):
        for (M, N, K) in shapes_for(c):
            A, B = synthetic.gemm_inputs(M, N, K, seed=M + 7 * N + 13 * K)
            case = DeviceCase(A, B, bcm)
            if c.family == 0 and M % c.block_m == 0 and N % c.block_n == 0 and K >= 6 * c.block_k:
                # the whole-tile unsplit pipelined kernel with nk > stages
                p = plan_of(case, c.id)
                assert (p.form, p.splits) == (t.FORM_PIPELINED, 1), (c.id, M, N, K, p.as_dict())
                assert K // c.block_k > c.stages
                steady += 1
            check_case(case, f"with_config[{c.id}]", config=c.id)
    assert steady == 2 * sum(1 for c in table(t) if c.family == 0)


EDGE_MN = [1, 15, 16, 17, 31, 32, 33, 255, 256, 257]
EDGE_K = [0, 1, 4, 27, 63, 64, 65, 777]
# the exhaustive grid adds multiples of 16 that no tile divides: ragged tiles
# of the unpredicated kernels
EXH_MN = EDGE_MN + [48, 272]
EXH_K = EDGE_K + [16, 48, 752]


@pytest.mark.parametrize("bcm", [True, False])
def test_edge_grid_sample_every_config(lib, bcm):
    """Every compiled configuration forced on a seeded sample of the edge
    grid M, N in EDGE_MN x K in EDGE_K (24 shapes per configuration and
    layout, different per configuration), with padded leading dimensions on
    every other shape."""
    t = lib
    grid = [(m, n, k) for m in EDGE_MN for n in EDGE_MN for k in EDGE_K]
    for c in table(t):
        rng = np.random.default_rng(1000 + c.id + (0 if bcm else 500))
        for i, gi in enumerate(rng.choice(len(grid), 24, replace=False)):
            M, N, K = grid[gi]
            A, B = synthetic.gemm_inputs(M, N, K, seed=int(gi))
            if i % 2:
                case = DeviceCase(A, B, bcm, lda=max(K, 1) + 3, ldb=(max(K, 1) if bcm else max(N, 1)) + 5, ldc=N + 2)
            else:
                case = DeviceCase(A, B, bcm)
            if K == 0:
                check_case(case, f"edge cfg{c.id}", config=c.id, expect=np.zeros((M, N), np.int32))
            else:
                check_case(case, f"edge cfg{c.id}", config=c.id)


@pytest.mark.parametrize("aligned", [False, True])
@pytest.mark.parametrize("bcm", [True, False])
def test_edge_grid_exhaustive_every_config(lib, bcm, aligned):
    """Every compiled configuration on the whole edge grid (M, N in EXH_MN,
    K in EXH_K: 1584 shapes).  The operands are top-left corners of one large
    matrix each, so every row carries real (nonzero) bytes past K (past N for
    row-major B) that must not enter the sum.  Unaligned: lda = 781 and ldb =
    781 or 261 (predicated kernels throughout); aligned: lda = 784 and ldb =
    784 or 272, so tile-multiple shapes take the unpredicated kernels.  Each shape writes its own C region (ldc =
    N + 2) inside one sentinel-filled buffer; the padding and the gaps
    between regions must survive.  All launches of a configuration go out
    before one synchronisation."""
    import oracle
    t = lib
    Mx, Kx = max(EXH_MN), max(EXH_K)
    A, B = synthetic.gemm_inputs(Mx, Mx, Kx, seed=77)
    pad = (lambda w: (w + 15) // 16 * 16 - w) if aligned else (lambda w: 4)
    lda = Kx + pad(Kx)
    A_st = np.zeros((Mx, lda), np.int8)
    A_st[:, :Kx] = A
    A_st[:, Kx:] = 55
    Bs = synthetic.store_b(B, bcm)
    ldb = Bs.shape[1] + pad(Bs.shape[1])
    B_st = np.zeros((Bs.shape[0], ldb), np.int8)
    B_st[:, :Bs.shape[1]] = Bs
    B_st[:, Bs.shape[1]:] = -55
    shapes = [(m, n, k) for m in EXH_MN for n in EXH_MN for k in EXH_K]
    want, offs, total = {}, {}, 0
    for (m, n, k) in shapes:
        want[(m, n, k)] = oracle.gemm(A_st[:m], B_st[:(n if bcm else k)], bcm, M=m, N=n, K=k)
        offs[(m, n, k)] = total
        total += m * (n + 2) + 16
    Ad = torch.from_numpy(A_st).cuda()
    Bd = torch.from_numpy(B_st).cuda()
    Cd = torch.empty(total, dtype=torch.int32, device="cuda")
    for c in table(t):
        note(f"[case] exhaustive edge grid cfg{c.id} bcm={bcm} lda={lda} ldb={ldb}")
        Cd.fill_(-123456789)
        for (m, n, k) in shapes:
            st = t.gemm_s8s8s32_with_config(c.id, int(bcm), m, n, k, Ad.data_ptr(), lda, Bd.data_ptr(), ldb,
                                            Cd.data_ptr() + 4 * offs[(m, n, k)], n + 2, 0)
            assert st == t.OK, (c.id, m, n, k, t.tdi8_status_string(st))
        torch.cuda.synchronize()
        flat = Cd.cpu().numpy()
        for (m, n, k) in shapes:
            o = offs[(m, n, k)]
            reg = flat[o:o + m * (n + 2)].reshape(m, n + 2)
            if not np.array_equal(reg[:, :n], want[(m, n, k)]):
                bad = np.argwhere(reg[:, :n] != want[(m, n, k)])
                raise AssertionError(f"cfg{c.id} {m}x{n}x{k} bcm={bcm}: {len(bad)} mismatches, first {bad[0]}")
            assert (reg[:, n:] == -123456789).all(), f"cfg{c.id} {m}x{n}x{k}: ldc padding written"
            assert (flat[o + m * (n + 2):o + m * (n + 2) + 16] == -123456789).all(), f"cfg{c.id} {m}x{n}x{k}: gap written"


def test_split_k_deterministic(lib):
    """The K-split form adds partial tiles with atomics in whatever order the
    blocks finish; integer addition makes the bytes identical every time."""
    t = lib
    M, N, K = 256, 256, 32768
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert t.tile_config_split_k(t.select_tile_config(M, N, K), M, N, K, cus) > 1
    A, B = synthetic.gemm_inputs(M, N, K, seed=21)
    case = DeviceCase(A, B, True)
    first = None
    for _ in range(5):
        case.c_buf.fill_(-123456789)
        assert case.run(None) == t.OK
        C, _ = case.result()
        first = C if first is None else first
        assert np.array_equal(C, first)
    assert np.array_equal(first, case.oracle())


def test_skinny_row_major_column_groups(lib):
    """Row-major B on a skinny configuration: with N and K multiples of 16 and
    N whole 128-column groups or more than two of them, a block covers 128
    columns (the last group may end at N) over one of G =
    128 / block width K slices of whole 16-byte chunks (slices differ by at
    most one chunk, empty when K / 16 < G; a slice may end inside a K tile)
    and adds into a zeroed
    C; otherwise the predicated form runs.  Both must equal the oracle, and
    the ldc padding must survive the zeroing."""
    t = lib
    for c in table(t):
        if c.family != 1:
            continue
        G = 128 // c.block_n
        kt = G * (512 if c.block_m == 16 else 256)
        for (M, N, K, ldc_pad) in [(c.block_m, 128, kt, 0), (2 * c.block_m, 384, 2 * kt, 8),
                                   (c.block_m, 256, 3 * kt, 4), (c.block_m, 128, kt + c.block_k, 0),
                                   (c.block_m, 128, 16 * G * 5, 0), (c.block_m - 3, 256, 16 * G * 37, 4),
                                   (c.block_m, 128 + c.block_n, 16 * G * 37, 0),
                                   (c.block_m, 128 + c.block_n, 1000, 0),
                                   # K slices of unequal length, and empty ones
                                   (c.block_m, 256, 16 * G * 5 + 48, 0), (c.block_m, 128, 16, 0),
                                   (2 * c.block_m - 1, 384, 4000, 8),
                                   # a last group that ends inside its 128 columns
                                   (c.block_m, 400, 16 * G * 5 + 48, 4)]:
            A, B = synthetic.gemm_inputs(M, N, K, seed=M + N + K + c.id)
            check_case(DeviceCase(A, B, False, ldc=N + ldc_pad), f"rr groups cfg{c.id}", config=c.id)


@pytest.mark.parametrize("bcm", [True, False])
def test_split_k_every_general_config(lib, bcm):
    """One tile and a long K: the unpredicated form splits K into slices whose
    partial sums are added into a zeroed C; bytes must equal the oracle's."""
    t = lib
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    for c in table(t):
        if c.family != 0:
            continue
        for (M, N, K) in [(c.block_m, c.block_n, 32 * c.block_k), (2 * c.block_m, c.block_n, 16 * c.block_k)]:
            s = t.tile_config_split_k(c.id, M, N, K, cus)
            assert s >= 2, (c.id, M, N, K, s)
            A, B = synthetic.gemm_inputs(M, N, K, seed=M + N + K)
            for ldc in (N, N + 8):   # ldc padding must stay untouched by the zeroing kernel
                case = DeviceCase(A, B, bcm, ldc=ldc)
                p = plan_of(case, c.id)
                assert (p.form, p.splits, p.kernels) == (t.FORM_SPLIT, s, 2), (c.id, M, N, K, p.as_dict())
                check_case(case, f"split-K x{s} cfg{c.id} ldc={ldc}", config=c.id)


@pytest.mark.parametrize("bcm", [True, False])
def test_split_k_edge_form_every_general_config(lib, bcm):
    """The K split of the edge form: M and N ending inside a tile (N any
    width with column-major B), K slices of whole 16-byte chunks that end
    inside K tiles and differ by one chunk, and whole tiles whose K does not
    split into whole K tiles.  Bytes must equal the oracle's; C's padding
    (past a partial group of four columns too) must survive the zeroing."""
    t = lib
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    for c in table(t):
        if c.family != 0:
            continue
        bm, bn, bk = c.block_m, c.block_n, c.block_k
        nr = bn + (5 if bcm else 16)
        for (M, N, K, pad) in [(bm + 7, nr, 33 * bk + 16, 0), (bm - 1, nr, 16 * 271, 3),
                               (bm, bn, 25 * bk, 4), (bm, bn, 17 * bk + 48, 0), (2 * bm + 1, 2 * bn, 16 * bk + 16, 8)]:
            s = t.tile_config_split_k(c.id, M, N, K, cus)
            assert s >= 2, (c.id, M, N, K, s)
            ldc = N + pad
            ldc += -ldc % 4   # a multiple of 4, as the unpredicated path needs
            A, B = synthetic.gemm_inputs(M, N, K, seed=M + N + K + c.id)
            case = DeviceCase(A, B, bcm, ldc=ldc)
            p = plan_of(case, c.id)
            whole = M % bm == 0 and N % bn == 0 and K % (s * bk) == 0
            assert p.form == (t.FORM_SPLIT if whole else t.FORM_SPLIT_EDGE) and p.splits == s, (c.id, M, N, K, p.as_dict())
            check_case(case, f"edge split-K x{s} cfg{c.id} {M}x{N}x{K}", config=c.id)


@pytest.mark.parametrize("bcm", [True, False])
def test_split_k_selected_long_k_shapes(lib, bcm):
    t = lib
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    for (M, N, K) in [(256, 256, 32768), (1024, 1024, 8192), (128, 256, 65536), (64, 128, 131072),
                      (500, 496, 16384), (1000, 1008, 8192), (300, 304, 32768 + 16)]:
        cid = t.select_tile_config(M, N, K)
        note(f"[info] {M}x{N}x{K} config {cid} splits {t.tile_config_split_k(cid, M, N, K, cus)}")
        A, B = synthetic.gemm_inputs(M, N, K, seed=11)
        check_case(DeviceCase(A, B, bcm), "selected long K")
    # all -128 at K = 131072 wraps to -2^31 exactly; split slices must wrap the same way
    M, N, K = 64, 128, 131072
    lo = np.full((M, K), -128, np.int8)
    lob = np.full((K, N), -128, np.int8)
    check_case(DeviceCase(lo, lob, bcm), "split wrap", expect=np.full((M, N), -(2 ** 31), np.int32))


@pytest.mark.parametrize("bcm", [True, False])
def test_identity_and_permutation_layout_probe(lib, bcm):
    """A = I gives C = B and A = P gives permuted rows of B: pins the
    accumulator-to-(row, column) map of every configuration."""
    t = lib
    rng = np.random.default_rng(0)
    for c in table(t):
        K = 64 if c.family == 1 else c.block_k
        M = K
        N = max(c.block_n, 64)
        B = rng.integers(-128, 128, size=(K, N)).astype(np.int8)
        eye = np.eye(K, dtype=np.int8)
        check_case(DeviceCase(eye, B, bcm), f"identity cfg{c.id}", config=c.id, expect=B.astype(np.int32))
        perm = rng.permutation(K)
        check_case(DeviceCase(eye[perm], B, bcm), f"perm cfg{c.id}", config=c.id,
                   expect=B[perm].astype(np.int32))


@pytest.mark.parametrize("bcm", [True, False])
def test_padded_and_misaligned_operands(lib, bcm):
    t = lib
    M, N, K = 70, 90, 150
    A, B = synthetic.gemm_inputs(M, N, K, seed=4)
    bk = N if not bcm else K
    for c in table(t):
        for (lda, ldb, ldc, offs) in [(K + 1, bk + 3, N + 1, (0, 0, 0)), (K + 16, bk + 16, N + 4, (1, 2, 1)),
                                      (K, bk, N, (3, 5, 2)), (K + 32, bk + 64, N + 8, (16, 16, 4))]:
            case = DeviceCase(A, B, bcm, lda=lda, ldb=ldb, ldc=ldc, offsets=offs)
            check_case(case, f"padded cfg{c.id} offs={offs}", config=c.id)


@pytest.mark.parametrize("bcm", [True, False])
def test_selected_entry_edge_shapes(lib, bcm):
    for (M, N, K) in [(1, 1, 1), (1, 4096, 4096), (32, 4096, 256), (33, 100, 1000), (16, 8192, 512),
                      (4096, 16, 300), (257, 255, 64), (512, 512, 27), (300, 300, 4)]:
        A, B = synthetic.gemm_inputs(M, N, K, seed=9)
        check_case(DeviceCase(A, B, bcm), "selected")


@pytest.mark.parametrize("bcm", [True, False])
def test_zero_sizes(lib, bcm):
    t = lib
    # K = 0: the C window becomes 0, padding untouched
    A = np.zeros((5, 0), np.int8)
    B = np.zeros((0, 7), np.int8)
    case = DeviceCase(A, B, bcm, lda=1, ldb=1 if bcm else 7, ldc=9)
    check_case(case, "K=0", expect=np.zeros((5, 7), np.int32))
    for cid in range(t.tile_config_count()):
        case = DeviceCase(A, B, bcm, lda=1, ldb=1 if bcm else 7, ldc=9)
        check_case(case, f"K=0 cfg{cid}", config=cid, expect=np.zeros((5, 7), np.int32))
    # M = 0 / N = 0: nothing is written
    for (M, N) in [(0, 5), (5, 0)]:
        A, B = synthetic.gemm_inputs(M, N, 8, seed=1)
        case = DeviceCase(A, B, bcm, ldc=max(N, 1))
        assert case.run(None) == t.OK
        _, rest = case.result()
        assert (rest == -123456789).all()


def test_extreme_values_closed_forms(lib):
    for bcm in (True, False):
        for (M, N, K) in [(256, 256, 256), (16, 4096, 4096), (100, 50, 777)]:
            lo = np.full((M, K), -128, np.int8)
            lob = np.full((K, N), -128, np.int8)
            check_case(DeviceCase(lo, lob, bcm), "all -128", expect=np.full((M, N), 16384 * K, np.int32))
            hi = np.full((M, K), 127, np.int8)
            check_case(DeviceCase(hi, lob, bcm), "127 x -128", expect=np.full((M, N), -16256 * K, np.int32))


def test_deterministic_bytes(lib):
    A, B = synthetic.gemm_inputs(1000, 3000, 777, seed=0)
    case = DeviceCase(A, B, True)
    first = None
    for _ in range(5):
        case.c_buf.fill_(-123456789)
        assert case.run(None) == lib.OK
        C, _ = case.result()
        first = C if first is None else first
        assert np.array_equal(C, first)


def test_non_default_stream(lib):
    A, B = synthetic.gemm_inputs(256, 256, 256, seed=3)
    case = DeviceCase(A, B, False)
    s = torch.cuda.Stream()
    note("[case] stream launch 256^3")
    with torch.cuda.stream(s):
        assert case.run(None, stream=s.cuda_stream) == lib.OK
    s.synchronize()
    C, rest = case.result()
    assert np.array_equal(C, case.oracle()) and (rest == -123456789).all()


def test_graph_capture_and_replay(lib):
    """The entry points only enqueue kernels (no allocation, no memset), so a
    call can be captured into a HIP graph.  Every replay, with eager work and
    synchronisations in between, must reproduce the eager bytes: the plain
    form, the K split (zero-fill kernel then split kernel) and the row-major
    skinny column groups (also zero fill then split)."""
    t = lib
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    for (M, N, K, bcm) in [(512, 512, 1024, True), (256, 256, 32768, True), (16, 4096, 4096, False)]:
        note(f"[case] graph capture {M}x{N}x{K} bcm={bcm} config={t.select_tile_config(M, N, K)} "
             f"splits={t.tile_config_split_k(t.select_tile_config(M, N, K), M, N, K, cus)}")
        A, B = synthetic.gemm_inputs(M, N, K, seed=5)
        Ad = torch.from_numpy(A).cuda()
        Bd = torch.from_numpy(synthetic.store_b(B, bcm)).cuda()
        want = t.gemm(Ad, Bd, bcm)
        torch.cuda.synchronize()
        assert np.array_equal(want.cpu().numpy(), oracle_gemm(A, B))
        out = torch.empty((M, N), dtype=torch.int32, device="cuda")
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            t.gemm(Ad, Bd, bcm, out=out)          # warm-up on the capture stream
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            t.gemm(Ad, Bd, bcm, out=out)
        for r in range(4):
            out.fill_(-7)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(out, want), f"replay {r}"
            t.gemm(Ad, Bd, bcm)                   # eager work between replays
            torch.cuda.synchronize()


def oracle_gemm(A, B):
    import oracle
    return oracle.gemm(A, B, False)


def test_block_per_cu_matches_occupancy_query(lib):
    """Claim 6's block_per_cu as the oracle computes it (register and LDS
    quotients on CDNA4's limits, from the registers and LDS the build read out
    of each kernel) equals the runtime's occupancy query on the device, for
    every compiled configuration; the limits themselves are the device's."""
    from oracle.selector import CuLimits, block_per_cu
    t = lib
    props = torch.cuda.get_device_properties(0)
    assert props.gcnArchName.startswith("gfx950")
    lim = CuLimits()
    note(f"[info] device: {props.max_threads_per_multi_processor} threads per CU "
         f"(limits assume {lim.simds * lim.wave_slots * lim.wave_size}), "
         f"{props.regs_per_multiprocessor} registers per CU")
    got, want = [], []
    for c in table(t):
        got.append(c.blocks_per_cu)
        want.append(block_per_cu(c.vgprs, c.agprs, c.lds_bytes, c.threads, lim))
    note(f"[info] occupancy query {got}; claim 6 {want}; "
         f"registers {[(c.vgprs, c.agprs) for c in table(t)]}")
    assert got == want


def test_selection_on_device_matches_oracle(lib):
    from oracle.selector import Cfg, Hw, block_per_cu, select
    t = lib
    props = torch.cuda.get_device_properties(0)
    assert props.gcnArchName.startswith("gfx950")
    tab = table(t)
    fam = {0: "general", 1: "skinny"}
    # the oracle's own block_per_cu (claim 6), not the library's occupancy query
    otab = [Cfg(c.id, fam[c.family], c.mfma_m, c.mfma_n, c.waves_m, c.waves_n, c.m_tiles, c.n_tiles,
                c.block_k, c.threads, block_per_cu(c.vgprs, c.agprs, c.lds_bytes, c.threads), c.stages,
                bool(c.excluded)) for c in tab]
    assert all(c.blocks_per_cu >= 1 for c in otab)
    hw = Hw(num_cu=props.multi_processor_count, max_threads_per_block=1024, min_active_threads=256,
            skinny_max_m=32)
    for (M, N, K) in [(256, 256, 256), (4096, 4096, 4096), (16, 4096, 4096), (1000, 3000, 777),
                      (16384, 16384, 8192), (1, 1, 1), (33, 4096, 4096)]:
        want = select(M, N, K, hw, otab)
        assert t.select_tile_config(M, N, K) == want.id, (M, N, K, want.trace)
    note(f"[info] device CUs={props.multi_processor_count} "
         f"bpc={[c.blocks_per_cu for c in tab]} regs={[c.vgprs for c in tab]}")


def test_plan_of_the_workloads(lib):
    """The kernel form gemm_plan reports for the five workload shapes with
    tight, allocation-aligned operands (what the bench and the workload
    tests run)."""
    t = lib
    cases = [((256, 256, 256), False, t.FORM_PIPELINED), ((4096, 4096, 4096), True, t.FORM_PIPELINED),
             ((4096, 4096, 4096), False, t.FORM_PIPELINED), ((16, 4096, 4096), True, t.FORM_SKINNY_DMA),
             ((16, 4096, 4096), False, t.FORM_SKINNY_ROW_GROUPS), ((1000, 3000, 777), True, t.FORM_PREDICATED),
             ((1000, 3000, 777), False, t.FORM_PREDICATED), ((16384, 16384, 8192), True, t.FORM_PIPELINED)]
    base = 1 << 30   # 16-byte aligned addresses standing in for allocations; nothing is dereferenced
    for (M, N, K), bcm, form in cases:
        p = t.gemm_plan(-1, bcm, M, N, K, base, K, base + (1 << 32), K if bcm else N, base + (1 << 36), N)
        note(f"[info] plan {M}x{N}x{K} bcm={bcm}: {p.as_dict()}")
        assert p.config_id == t.select_tile_config(M, N, K) and p.form == form, (M, N, K, bcm, p.as_dict())


def test_predicated_fill_plan(lib):
    """Calls whose operands take the predicated kernels with column-major B
    run the configuration the oracle's predicated_fill gives for the
    selection's pick (more tiles when the pick leaves compute units idle),
    gemm_plan reports it, row-major B and forced ids are left alone, and the
    results are bit-exact."""
    from oracle.selector import Cfg, predicated_fill
    t = lib
    tab = table(t)
    fam = {0: "general", 1: "skinny"}
    otab = [Cfg(c.id, fam[c.family], c.mfma_m, c.mfma_n, c.waves_m, c.waves_n, c.m_tiles, c.n_tiles,
                c.block_k, c.threads, c.blocks_per_cu, c.stages, bool(c.excluded)) for c in tab]
    import torch
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    moved = 0
    for (M, N, K) in [(1000, 1000, 8191), (512, 512, 4097), (333, 777, 999), (1000, 3000, 777), (900, 900, 1001),
                      (40, 700, 300)]:
        A, B = synthetic.gemm_inputs(M, N, K, seed=M + N)
        sel = t.select_tile_config(M, N, K)
        for bcm in (True, False):
            case = DeviceCase(A, B, bcm, lda=K + 1, ldb=(K if bcm else N) + 1)
            p = plan_of(case)
            want = predicated_fill(otab[sel], M, N, cus, otab).id if (bcm and tab[sel].family == 0) else sel
            assert p.config_id == want, (M, N, K, bcm, sel, p.as_dict())
            assert plan_of(case, sel).config_id == sel
            moved += want != sel
            if M * N * K <= 1000 * 1000 * 8191 // 4 or want != sel:
                check_case(case, f"predicated fill {M}x{N}x{K} bcm={bcm} cfg{p.config_id}")
    assert moved >= 3


# ---- the five workloads -------------------------------------------------------------

def sampled_check(C_dev, A_store, B_store, bcm, M, N, K, seed, n_random=4096, freivalds=2):
    import oracle
    rng = np.random.default_rng(seed)
    rows = np.concatenate([np.zeros(N, np.int64), np.full(N, M - 1), np.arange(M), np.arange(M),
                           rng.integers(0, M, n_random)])
    cols = np.concatenate([np.arange(N), np.arange(N), np.zeros(M, np.int64), np.full(M, N - 1),
                           rng.integers(0, N, n_random)])
    C = C_dev.cpu().numpy()
    want = oracle.gemm_elements(A_store, B_store, bcm, K, rows, cols)
    got = C[rows, cols]
    assert np.array_equal(got, want), f"{int((got != want).sum())} sampled mismatches"
    if freivalds:
        # exact in float64: every partial sum is an integer below 2**53
        X = synthetic.freivalds_vectors(N, freivalds, seed).astype(np.float64)
        B_log = B_store[:N, :K].T if bcm else B_store[:K, :N]
        BX = np.zeros((K, freivalds))
        for k0 in range(0, K, 2048):
            BX[k0:k0 + 2048] = B_log[k0:k0 + 2048].astype(np.float64) @ X.T
        for m0 in range(0, M, 2048):
            left = C[m0:m0 + 2048].astype(np.float64) @ X.T
            right = A_store[m0:m0 + 2048, :K].astype(np.float64) @ BX
            assert np.array_equal(left, right), f"Freivalds mismatch in rows {m0}.."


WORKLOADS = {
    "cfg1_256": (256, 256, 256),
    "cfg2_4096": (4096, 4096, 4096),
    "cfg3_skinny": (16, 4096, 4096),
    "cfg4_ragged": (1000, 3000, 777),
}


@pytest.mark.parametrize("name", list(WORKLOADS))
@pytest.mark.parametrize("bcm", [True, False])
def test_workloads_seeds(lib, name, bcm):
    M, N, K = WORKLOADS[name]
    for seed in (0, 1, 2):
        A, B = synthetic.gemm_inputs(M, N, K, seed)
        case = DeviceCase(A, B, bcm)
        cfg = lib.select_tile_config(M, N, K)
        note(f"[case] {name} seed={seed} bcm={bcm} selected={cfg}")
        # every element against the oracle (4096^3: ~1.5 s of the oracle on the host's cores)
        check_case(case, f"{name} seed {seed}")
        if M * N * K > 4 * 10 ** 9:
            # and the sampled and Freivalds checks of the same output, as extras
            win = case.c_buf[:M * N].view(M, N)
            sampled_check(win, case.A_store, case.B_store, bcm, M, N, K, seed)


_LARGE = {}


def large_inputs_and_oracle():
    """Seed-0 operands of the 16384 x 16384 x 8192 workload and the oracle's
    C for them, computed once (about a minute on the host's cores) and shared
    by both B layouts: the generator fills the logical matrices, so both
    layouts of one seed have the same product."""
    if "C" not in _LARGE:
        import time
        import oracle
        M, N, K = 16384, 16384, 8192
        note("[case] cfg5 16384x16384x8192 generating seed 0")
        A, B = synthetic.gemm_inputs(M, N, K, 0)
        Bs = synthetic.store_b(B, True)
        note(f"[case] cfg5 oracle on {oracle.num_threads()} threads")
        t0 = time.perf_counter()
        _LARGE["C"] = oracle.gemm(A, Bs, True, M=M, N=N, K=K)
        note(f"[case] cfg5 oracle done in {time.perf_counter() - t0:.1f} s")
        _LARGE["A"], _LARGE["B"] = A, B
    return _LARGE["A"], _LARGE["B"], _LARGE["C"]


@pytest.mark.parametrize("bcm", [True, False])
def test_workload_large_16384(lib, bcm):
    """Every element of the 16384 x 16384 x 8192 product against the oracle,
    both B layouts, seed 0, from the selected call and from the persistent
    form; C sits in a sentinel-filled buffer whose canary after the last row
    must survive."""
    M, N, K = 16384, 16384, 8192
    A, B, want = large_inputs_and_oracle()
    Bs = synthetic.store_b(B, bcm)
    A_dev = torch.from_numpy(A).cuda()
    B_dev = torch.from_numpy(Bs).cuda()
    del Bs
    C_buf = torch.full((M * N + 64,), -123456789, dtype=torch.int32, device="cuda")
    C_dev = C_buf[:M * N].view(M, N)
    note(f"[case] cfg5 launch bcm={bcm} selected={lib.select_tile_config(M, N, K)}")
    lib.gemm(A_dev, B_dev, bcm, out=C_dev)
    torch.cuda.synchronize()
    got = C_dev.cpu().numpy()
    if not np.array_equal(got, want):
        bad = np.argwhere(got != want)
        raise AssertionError(f"cfg5 bcm={bcm}: {len(bad)} mismatches, first at {tuple(bad[0])}")
    assert (C_buf[M * N:].cpu().numpy() == -123456789).all(), "wrote past C"
    # the persistent form of the same configuration: 16 tiles per block
    note(f"[case] cfg5 persistent launch bcm={bcm}")
    C_buf.fill_(-123456789)
    lib.gemm(A_dev, B_dev, bcm, out=C_dev, persistent_blocks=0)
    torch.cuda.synchronize()
    del A_dev, B_dev
    got = C_dev.cpu().numpy()
    if not np.array_equal(got, want):
        bad = np.argwhere(got != want)
        raise AssertionError(f"cfg5 persistent bcm={bcm}: {len(bad)} mismatches, first at {tuple(bad[0])}")
    assert (C_buf[M * N:].cpu().numpy() == -123456789).all(), "persistent form wrote past C"
    del got, C_buf, C_dev
    torch.cuda.empty_cache()


@pytest.mark.parametrize("bcm", [True, False])
def test_int32_limit_and_wrap(lib, bcm):
    """All -128 operands at the largest K without overflow, and one step past
    it: the result is defined mod 2^32 (what int32 accumulation gives), so
    16384 * 131073 must wrap to its two's-complement value, not saturate."""
    t = lib
    for K in (131071, 131073):
        exact = 16384 * K
        want = ((exact + 2 ** 31) % 2 ** 32) - 2 ** 31
        for (M, N) in [(16, 64), (64, 128)]:
            A = np.full((M, K), -128, np.int8)
            B = np.full((K, N), -128, np.int8)
            C = check_case(DeviceCase(A, B, bcm), f"K={K} all -128", expect=np.full((M, N), want, np.int32))
            assert int(C[0, 0]) == want
        # and through a general-family configuration
        A = np.full((64, K), -128, np.int8)
        B = np.full((K, 128), -128, np.int8)
        check_case(DeviceCase(A, B, bcm), f"K={K} cfg7", config=7, expect=np.full((64, 128), want, np.int32))


@pytest.mark.parametrize("bcm", [True, False])
def test_long_k_random(lib, bcm):
    """Random operands over a long K (many K tiles and skinny chunks)."""
    for (M, N, K) in [(16, 256, 65536), (256, 256, 32768), (33, 70, 20000)]:
        A, B = synthetic.gemm_inputs(M, N, K, seed=5)
        check_case(DeviceCase(A, B, bcm), f"long K {M}x{N}x{K}")


def prefetch_fits(c):
    """The tile fits the deep-prefetch loop: whole 16-byte loads per thread,
    at most four per thread and K tile for A and B together."""
    a, b = c.block_m * c.block_k // 16, c.block_n * c.block_k // 16
    return a % c.threads == 0 and b % c.threads == 0 and a // c.threads + b // c.threads <= 4


@pytest.mark.parametrize("bcm", [True, False])
def test_predicated_deep_prefetch_boundaries(lib, bcm):
    """The predicated kernels (odd leading dimensions, misaligned pointers)
    of every general configuration at K around the deep-prefetch loop's
    bounds: fewer than three K tiles, a whole number of K tiles, one byte
    more, several groups of tiles in flight, tails of 1 to 16 bytes, with
    real bytes past K in every row and ragged M and N (edge rows read a
    clamped row).  The deep loop runs for column-major B whenever the tile
    fits it and the grid has at most one block per compute unit."""
    t = lib
    deep = 0
    for c in table(t):
        if c.family != 0:
            continue
        BK = c.block_k
        ks = sorted({16, 2 * BK + 5, 3 * BK, 4 * BK, 4 * BK + 1, 5 * BK, 5 * BK + 9, 8 * BK + 15, 9 * BK + 16,
                     17 * BK + 7})
        for i, K in enumerate(ks):
            M, N = c.block_m + 5 + i, 2 * c.block_n - 3
            A, B = synthetic.gemm_inputs(M, N, K, seed=31 * c.id + i)
            case = DeviceCase(A, B, bcm, lda=K + 1 + 2 * (i % 3), ldb=(K if bcm else N) + 3,
                              offsets=(1 + i % 5, 3, 0))
            p = plan_of(case, c.id)
            want = bcm and prefetch_fits(c) and -(-K // BK) >= 3
            assert p.form == (t.FORM_PREDICATED_PREFETCH if want else t.FORM_PREDICATED), (c.id, K, p.as_dict())
            deep += want
            check_case(case, f"predicated cfg{c.id} form {p.form}", config=c.id)
    assert deep > 0 or not bcm


def test_predicated_prefetch_only_for_small_grids(lib):
    """The same K and configuration on a grid of at most one block per
    compute unit (deep-prefetch loop) and on a larger one (the other loop):
    both bit-exact."""
    t = lib
    c = table(t)[t.select_tile_config(1000, 3000, 777)]
    assert prefetch_fits(c)
    for (M, N) in [(600, 1000), (1000, 3000)]:
        K = 777
        A, B = synthetic.gemm_inputs(M, N, K, seed=M)
        case = DeviceCase(A, B, True)
        p = plan_of(case, c.id)
        blocks = -(-M // c.block_m) * -(-N // c.block_n)
        assert p.form == (t.FORM_PREDICATED_PREFETCH if blocks <= 256 else t.FORM_PREDICATED), p.as_dict()
        check_case(case, f"predicated {M}x{N}x{K} form {p.form}", config=c.id)
