"""Persistent whole-tile form (gemm_s8s8s32_persistent) against the CPU
oracle, through the C ABI: every general configuration, both B layouts,
block counts that give every block one tile, several tiles, or unequal
numbers of tiles, K tile streams shorter and longer than the pipeline,
K = 0, and the 4096^3 workload in full.  Bit-exact on every element; C
sits in a sentinel-filled buffer that must survive outside the window."""
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


def general(t):
    return [c for c in (t.tile_config_info(i) for i in range(t.tile_config_count())) if c.family == 0]


def cases_for(c):
    BM, BN, BK = c.block_m, c.block_n, c.block_k
    return [
        ((BM, BN, BK), 0),            # one tile, one K tile (shorter than the pipeline)
        ((2 * BM, 3 * BN, 5 * BK), 0),  # one tile per block, five K tiles
        ((2 * BM, 3 * BN, 5 * BK), 4),  # six tiles on four blocks: two blocks take two
        ((3 * BM, BN, 2 * BK), 1),    # one block walks three tiles of two K tiles
        ((2 * BM, 2 * BN, BK), 3),    # one K tile per tile: the stream crosses a tile every step
        ((BM, 4 * BN, 3 * BK), 2),    # two tiles per block along N
    ]


@pytest.mark.parametrize("bcm", [True, False])
def test_persistent_every_general_config(lib, bcm):
    t = lib
    for c in general(t):
        for (M, N, K), blocks in cases_for(c):
            A, B = synthetic.gemm_inputs(M, N, K, seed=M + 3 * N + 11 * K + blocks)
            case = DeviceCase(A, B, bcm)
            check_case(case, f"persistent[{c.id}] blocks={blocks}", config=c.id, persistent=blocks)


@pytest.mark.parametrize("bcm", [True, False])
def test_persistent_k_zero_and_padded(lib, bcm):
    """K = 0 stores zero tiles; padded leading dimensions (multiples of 16)
    keep the pads untouched."""
    t = lib
    c = t.tile_config_info(0)
    M, N = 2 * c.block_m, c.block_n
    A, B = synthetic.gemm_inputs(M, N, 0, seed=5)
    case = DeviceCase(A, B, bcm, lda=16, ldb=16 if bcm else N)
    check_case(case, "persistent K=0", config=0, persistent=1, expect=np.zeros((M, N), np.int32))
    M, N, K = c.block_m, 2 * c.block_n, 3 * c.block_k
    A, B = synthetic.gemm_inputs(M, N, K, seed=6)
    case = DeviceCase(A, B, bcm, lda=K + 32, ldb=(K + 48) if bcm else (N + 16), ldc=N + 4)
    check_case(case, "persistent padded", config=0, persistent=1)


def test_persistent_rejects_what_it_cannot_run(lib):
    t = lib
    c = t.tile_config_info(0)
    M, N, K = c.block_m, c.block_n, c.block_k
    A, B = synthetic.gemm_inputs(M + 1, N, K, seed=1)
    ragged = DeviceCase(A, B, True)
    assert ragged.run(None, config=0, persistent=0) == t.ERR_BAD_CONFIG
    A, B = synthetic.gemm_inputs(M, N, K, seed=2)
    case = DeviceCase(A, B, True, lda=K + 1)
    assert case.run(None, config=0, persistent=0) == t.ERR_BAD_CONFIG
    skinny = [x.id for x in (t.tile_config_info(i) for i in range(t.tile_config_count())) if x.family == 1]
    case = DeviceCase(A, B, True)
    assert case.run(None, config=skinny[0], persistent=0) == t.ERR_BAD_CONFIG
    assert case.run(None, config=0, persistent=-1) == t.ERR_INVALID_VALUE
    # nothing was written
    C, rest = case.result()
    assert (C == -123456789).all() and (rest == -123456789).all()


@pytest.mark.parametrize("bcm", [True, False])
def test_persistent_workload_4096(lib, bcm):
    """4096^3 in full against the oracle: one tile per block (the default
    grid of 256 blocks) and two tiles per block (128 blocks)."""
    M = N = K = 4096
    A, B = synthetic.gemm_inputs(M, N, K, 0)
    case = DeviceCase(A, B, bcm)
    want = case.oracle()
    for blocks in (0, 128):
        note(f"[case] persistent 4096^3 bcm={bcm} blocks={blocks}")
        case.c_buf.fill_(-123456789)
        check_case(case, f"persistent 4096^3 blocks={blocks}", persistent=blocks, expect=want)


@pytest.mark.parametrize("bcm", [True, False])
def test_persistent_random_cases(lib, bcm):
    """Seeded random whole-tile shapes for random general configurations:
    random tile counts along M and N, K tile counts from 1 to 9, block counts
    from 1 to past the tile count, leading dimensions padded by multiples of
    16 (ldc by multiples of 4) and operands offset by multiples of 16 bytes."""
    t = lib
    cfgs = general(t)
    rng = np.random.default_rng(20261203 + (1 if bcm else 0))
    for i in range(48):
        c = cfgs[int(rng.integers(0, len(cfgs)))]
        tm, tn, tk = (int(rng.integers(1, 5)), int(rng.integers(1, 5)), int(rng.integers(1, 10)))
        M, N, K = tm * c.block_m, tn * c.block_n, tk * c.block_k
        blocks = int(rng.integers(0, tm * tn + 3))
        lda = K + 16 * int(rng.integers(0, 3))
        ldb = (K if bcm else N) + 16 * int(rng.integers(0, 3))
        ldc = N + 4 * int(rng.integers(0, 3))
        offs = (16 * int(rng.integers(0, 2)), 16 * int(rng.integers(0, 2)), 4 * int(rng.integers(0, 2)))
        A, B = synthetic.gemm_inputs(M, N, K, seed=5000 + i)
        case = DeviceCase(A, B, bcm, lda=lda, ldb=ldb, ldc=ldc, offsets=offs)
        check_case(case, f"persistent random {i} config {c.id} blocks={blocks}", config=c.id, persistent=blocks)


def test_persistent_graph_capture_and_replay(lib):
    """The persistent entry point only enqueues its kernel, so a call can be
    captured into a HIP graph; every replay, with eager work in between,
    reproduces the oracle's bytes (two tiles per block)."""
    import oracle
    t = lib
    c = t.tile_config_info(0)
    M, N, K = 2 * c.block_m, 2 * c.block_n, 4 * c.block_k
    A, B = synthetic.gemm_inputs(M, N, K, seed=9)
    want = oracle.gemm(A, B, False)
    for bcm in (True, False):
        note(f"[case] persistent graph capture {M}x{N}x{K} bcm={bcm}")
        Ad = torch.from_numpy(A).cuda()
        Bd = torch.from_numpy(synthetic.store_b(B, bcm)).cuda()
        out = torch.empty((M, N), dtype=torch.int32, device="cuda")
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            t.gemm(Ad, Bd, bcm, out=out, config=0, persistent_blocks=2)   # warm-up on the capture stream
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            t.gemm(Ad, Bd, bcm, out=out, config=0, persistent_blocks=2)
        for r in range(4):
            out.fill_(-7)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert np.array_equal(out.cpu().numpy(), want), f"replay {r}"
            t.gemm(Ad, Bd, bcm)                   # eager work between replays
            torch.cuda.synchronize()
