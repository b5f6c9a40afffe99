"""Seeded random parity cases through the C ABI: shapes drawn to land on,
next to and between tile multiples, random leading-dimension padding
(aligned or not), random byte offsets of the operands, both B layouts, the
selected entry points and forced configurations.  Bit-exact against the
oracle; C's padding and the canary after it must keep their sentinel."""
import numpy as np
import pytest

import synthetic
from helpers import DeviceCase, check_case

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import tiled_dense_int8_amd as t
    return t


def draw_dim(rng, hi):
    kind = rng.integers(0, 5)
    if kind == 0:
        return int(rng.integers(1, 33))                  # skinny range
    if kind == 1:
        return int(16 * rng.integers(1, hi // 16 + 1))   # multiple of 16
    if kind == 2:
        m = int(64 * rng.integers(1, hi // 64 + 1))       # next to a tile multiple
        return max(1, m + int(rng.integers(-1, 2)))
    return int(rng.integers(1, hi + 1))


def draw_case(rng, bcm):
    M, N, K = draw_dim(rng, 600), draw_dim(rng, 600), draw_dim(rng, 800)
    aligned = rng.random() < 0.5
    if aligned:
        pad = lambda: int(16 * rng.integers(0, 3))
        offs = tuple(int(16 * rng.integers(0, 2)) for _ in range(2)) + (int(4 * rng.integers(0, 2)),)
    else:
        pad = lambda: int(rng.integers(0, 40))
        offs = tuple(int(rng.integers(0, 16)) for _ in range(3))
    lda = K + pad()
    ldb = (K if bcm else N) + pad()
    ldc = N + (int(4 * rng.integers(0, 3)) if aligned else int(rng.integers(0, 9)))
    return M, N, K, lda, ldb, ldc, offs


@pytest.mark.parametrize("bcm", [True, False])
def test_random_shapes_layouts_and_entries(lib, bcm):
    t = lib
    n_cfg = t.tile_config_count()
    rng = np.random.default_rng(20261202 + (1 if bcm else 0))
    for i in range(160):
        M, N, K, lda, ldb, ldc, offs = draw_case(rng, bcm)
        A, B = synthetic.gemm_inputs(M, N, K, seed=1000 + i)
        case = DeviceCase(A, B, bcm, lda=lda, ldb=ldb, ldc=ldc, offsets=offs)
        config = None if rng.random() < 0.6 else int(rng.integers(0, n_cfg))
        check_case(case, f"random[{i}] offs={offs}", config=config)


def test_random_convolutions(lib):
    """Seeded random convolution geometries (channels on both sides of the
    16-channel DMA form, padding, stride, dilation, filters up to 5 x 5),
    compared in full with the convolution oracle."""
    import oracle
    from test_gpu_conv import run_conv
    t = lib
    rng = np.random.default_rng(20261203)
    done = 0
    while done < 80:
        N = int(rng.integers(1, 4))
        H, W = int(rng.integers(1, 21)), int(rng.integers(1, 21))
        C = int(rng.choice([1, 3, 5, 8, 16, 17, 32, 48, 64]))
        K = int(rng.integers(1, 71))
        R, S = int(rng.integers(1, 6)), int(rng.integers(1, 6))
        pad = (int(rng.integers(0, 3)), int(rng.integers(0, 3)))
        stride = (int(rng.integers(1, 4)), int(rng.integers(1, 4)))
        dil = (int(rng.integers(1, 3)), int(rng.integers(1, 3)))
        if oracle.conv_out_extent(H, R, pad[0], stride[0], dil[0]) < 1 or \
                oracle.conv_out_extent(W, S, pad[1], stride[1], dil[1]) < 1:
            continue
        x, w = synthetic.conv_inputs(N, H, W, C, K, R, S, 500 + done)
        y, tail_ok = run_conv(t, x, w, pad, stride, dil, None, f"random[{done}]")
        want = oracle.conv2d(x, w, pad, stride, dil)
        assert np.array_equal(y, want), f"random[{done}]: {int((y != want).sum())} mismatches"
        assert tail_ok, f"random[{done}]: output tail overwritten"
        done += 1


@pytest.mark.parametrize("bcm", [True, False])
def test_random_k_split_shapes(lib, bcm):
    """Seeded random long-K shapes on aligned operands, where the K split
    runs: M and N on and off tile multiples (N any width with column-major
    B), K any multiple of 16 from 1024 to 16384 (slices ending inside K tiles,
    unequal by one chunk), padded leading dimensions, the selected or a
    forced general configuration.  Bit-exact against the oracle, and at
    least half of the cases must actually split."""
    t = lib
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    general = [c.id for c in (t.tile_config_info(i) for i in range(t.tile_config_count())) if c.family == 0]
    rng = np.random.default_rng(20261204 + (1 if bcm else 0))
    split_cases = 0
    for i in range(40):
        M = int(rng.integers(1, 201))
        N = int(rng.integers(1, 201)) if bcm else int(16 * rng.integers(1, 13))
        K = int(16 * rng.integers(64, 1025))
        config = None if rng.random() < 0.5 else int(rng.choice(general))
        cid = t.select_tile_config(M, N, K) if config is None else config
        s = t.tile_config_split_k(cid, M, N, K, cus)
        lda = K + int(16 * rng.integers(0, 3))
        ldb = (K if bcm else N) + int(16 * rng.integers(0, 3))
        ldc = N + int(4 * rng.integers(0, 3)) + (4 - N % 4) % 4
        A, B = synthetic.gemm_inputs(M, N, K, seed=3000 + i)
        case = DeviceCase(A, B, bcm, lda=lda, ldb=ldb, ldc=ldc)
        # count a case as split only if the call really runs a split kernel
        p = t.gemm_plan(-1 if config is None else config, bcm, M, N, K, case.A_ptr, lda, case.B_ptr, ldb,
                        case.C_ptr, ldc)
        assert p.config_id == cid and p.splits == s, (i, p.as_dict(), s)
        split_cases += p.form in (t.FORM_SPLIT, t.FORM_SPLIT_EDGE)
        check_case(case, f"random split[{i}] {M}x{N}x{K} cfg{cid} x{s}", config=config)
    assert split_cases >= 20, split_cases
