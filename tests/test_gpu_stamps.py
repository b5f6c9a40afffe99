"""The instrumented build (libtdi8_stamps.so, include/tdi8_stamps.h) computes
the same bytes as the library and writes one well-formed timeline record
per block: its block timelines are measurements of the product kernels."""
import os

import numpy as np
import pytest

import synthetic

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

# (M, N, K, B column-major): pipelined whole tiles, its edge form, a K split,
# the predicated kernel (odd leading dimensions), both skinny DMA layouts
CASES = [(512, 512, 1024, True), (300, 260, 512, True), (256, 256, 16384, True), (100, 300, 77, True),
         (16, 1024, 4096, True), (16, 1024, 4096, False), (200, 384, 640, False)]


@pytest.fixture(scope="module")
def libs():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import tiled_dense_int8_amd as t
    path = os.path.join(os.path.dirname(t.LIB_PATH), "libtdi8_stamps.so")
    s = t.load_library(path)
    import ctypes
    s.tdi8_stamps_set.argtypes = [ctypes.c_void_p, ctypes.c_int]
    s.tdi8_stamps_set.restype = ctypes.c_int
    yield t, s
    s.tdi8_stamps_set(None, 0)


@pytest.mark.parametrize("M,N,K,bcm", CASES)
def test_stamps_build_matches_library_and_records_every_block(libs, M, N, K, bcm):
    t, s = libs
    print(f"[stamps] {M}x{N}x{K} bcm={bcm}", flush=True)
    A, B = synthetic.gemm_inputs(M, N, K, seed=5)
    Bs = synthetic.store_b(B, bcm)
    a = torch.from_numpy(A).cuda()
    b = torch.from_numpy(Bs).cuda()
    args = lambda c: (M, N, K, a.data_ptr(), a.stride(0), b.data_ptr(), b.stride(0), c.data_ptr(), c.stride(0), 0)
    ref = torch.full((M, N), -7, dtype=torch.int32, device="cuda")
    got = torch.full((M, N), -7, dtype=torch.int32, device="cuda")
    plan = t.gemm_plan(-1, bcm, M, N, K, a.data_ptr(), a.stride(0), b.data_ptr(), b.stride(0), got.data_ptr(), N)
    blocks = plan.grid_x * plan.grid_y
    recs = torch.zeros((blocks + 8, 8), dtype=torch.int64, device="cuda")
    name = "gemm_s8s8s32_bt" if bcm else "gemm_s8s8s32"
    assert getattr(t, name)(*args(ref)) == t.OK
    assert s.tdi8_stamps_set(recs.data_ptr(), blocks) == t.OK
    assert getattr(s, name)(*args(got)) == t.OK
    assert s.tdi8_stamps_set(None, 0) == t.OK
    torch.cuda.synchronize()
    assert torch.equal(ref, got)
    r = recs.cpu().numpy()
    assert (r[blocks:] == 0).all(), "nothing past the capacity"
    r = r[:blocks]
    assert (r[:, 6] == np.arange(blocks)).all() and (r[:, 7] == 0).all()
    assert (r[:, 2] > r[:, 0]).all() and (r[:, 4] > r[:, 3]).all()
    loop = r[:, 1] > 0
    assert loop.all() or plan.splits > 1, "every block of an unsplit launch runs a K loop"
    assert ((r[loop, 1] >= r[loop, 0]) & (r[loop, 1] <= r[loop, 2])).all()
    ghz = (r[:, 2] - r[:, 0]).sum() / (r[:, 4] - r[:, 3]).sum() * 0.1
    assert 0.3 < ghz < 3.0, ghz
    assert len(set((r[:, 5] >> 32).tolist())) >= 1
