"""Operands whose last row starts past 2**31: the C ABI takes int sizes and
leading dimensions, but the products row * ld (and image * H * W * C) are
not ints.  Each kernel form runs with leading dimensions large enough that
A's and B's last rows start past 2**31 bytes and C's past 2**31 elements
(several GiB of device memory per case), on logical sizes the oracle
computes in full.  Bit-exact against the oracle; the padding of C around
the logical window must keep its sentinel."""
import numpy as np
import pytest

import synthetic
from helpers import note

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

SENT_A, SENT_B, SENT_C = 99, -77, -123456789
BIG = 2 ** 31


@pytest.fixture(scope="module")
def t():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import tiled_dense_int8_amd as lib
    return lib


def run_strided(t, desc, M, N, K, bcm, lda, ldb, ldc, seed, config=None):
    import oracle
    b_rows, b_cols = (N, K) if bcm else (K, N)
    assert (M - 1) * lda >= BIG and (b_rows - 1) * ldb >= BIG and (M - 1) * ldc >= BIG, "case too small"
    note(f"[case] {desc} M={M} N={N} K={K} bcm={bcm} lda={lda} ldb={ldb} ldc={ldc} config={config}")
    A, B = synthetic.gemm_inputs(M, N, K, seed)
    Bs = synthetic.store_b(B, bcm)
    a = torch.full((M, lda), SENT_A, dtype=torch.int8, device="cuda")
    a[:, :K].copy_(torch.from_numpy(A))
    b = torch.full((b_rows, ldb), SENT_B, dtype=torch.int8, device="cuda")
    b[:, :b_cols].copy_(torch.from_numpy(Bs))
    c = torch.full((M, ldc), SENT_C, dtype=torch.int32, device="cuda")
    args = (M, N, K, a.data_ptr(), lda, b.data_ptr(), ldb, c.data_ptr(), ldc, 0)
    if config is None:
        st = (t.gemm_s8s8s32_bt if bcm else t.gemm_s8s8s32)(*args)
    else:
        st = t.gemm_s8s8s32_with_config(config, bcm, *args)
    assert st == t.OK, t.tdi8_status_string(st)
    torch.cuda.synchronize()
    got = c[:, :N].cpu().numpy()
    pad_ok = bool((c[:, N:] == SENT_C).all().item())
    del a, b, c
    torch.cuda.empty_cache()
    want = oracle.gemm(A, Bs, bcm)
    assert np.array_equal(got, want), f"{desc}: {int((got != want).sum())} mismatches"
    assert pad_ok, f"{desc}: wrote into C's padding"


L23 = 2 ** 23                # 8 MiB rows
L23P = 2 ** 23 + 2 ** 20     # 9 MiB rows: 255 of them pass 2**31
L27P = 2 ** 27 + 2 ** 24     # 144 MiB rows: 15 of them pass 2**31


@pytest.mark.parametrize("bcm", [True, False])
def test_unpredicated_edge_form_large_ld(t, bcm):
    """Ragged M and N, aligned operands: the unpredicated kernel's edge form."""
    K = 256 if bcm else 320   # row-major B: K rows of ldb bytes
    run_strided(t, "edge form", 300, 272, K, bcm, L23, L23, L23, seed=11)


@pytest.mark.parametrize("bcm", [True, False])
def test_unpredicated_split_form_large_ld(t, bcm):
    """One 256 x 256 tile over a long K: the K-split form with atomics."""
    c = t.tile_config_info(0)
    assert (c.block_m, c.block_n) == (256, 256)
    num_cu = torch.cuda.get_device_properties(0).multi_processor_count
    assert t.tile_config_split_k(0, 256, 256, 4096, num_cu) > 1
    run_strided(t, "split form", 256, 256, 4096, bcm, L23P, L23P if bcm else 2 ** 19 + 2 ** 16, L23P, seed=12,
                config=0)


@pytest.mark.parametrize("bcm", [True, False])
def test_unpredicated_edge_split_form_large_ld(t, bcm):
    """Ragged M and N over a long K: the K split of the edge form."""
    num_cu = torch.cuda.get_device_properties(0).multi_processor_count
    cid = t.select_tile_config(300, 272, 4096)
    assert t.tile_config_split_k(cid, 300, 272, 4096, num_cu) > 1
    run_strided(t, "edge split form", 300, 272, 4096, bcm, L23, L23 if bcm else 2 ** 19 + 2 ** 16, L23, seed=16)


@pytest.mark.parametrize("bcm", [True, False])
def test_predicated_form_large_ld(t, bcm):
    """Odd leading dimensions: the predicated kernel."""
    run_strided(t, "predicated form", 300, 272, 300, bcm, L23 + 1, L23 + 3, L23 + 1, seed=13)


@pytest.mark.parametrize("bcm", [True, False])
def test_skinny_forms_large_ld(t, bcm):
    """M = 16: the skinny DMA kernel (column-major B) and the row-major
    column-group form."""
    if bcm:
        run_strided(t, "skinny", 16, 256, 2048, True, L27P, L23P, L27P, seed=14)
    else:
        run_strided(t, "skinny column groups", 16, 256, 4096, False, L27P, 2 ** 19 + 2 ** 16, L27P, seed=15)


CONV_BIG = (33, 256, 256, 1024, 16, 3, 3)   # N, H, W, C, K, R, S


@pytest.fixture(scope="module")
def conv_big_inputs():
    """Seeded image 0, last image and filters of CONV_BIG (host)."""
    N, H, W, C, K, R, S = CONV_BIG
    x0 = synthetic.uniform_int8(H * W, C, seed=21, tag=1).reshape(1, H, W, C)
    xl = synthetic.uniform_int8(H * W, C, seed=21, tag=2).reshape(1, H, W, C)
    w = synthetic.uniform_int8(K, R * S * C, seed=21, tag=3).reshape(K, R, S, C)
    return x0, xl, w


@pytest.mark.parametrize("misalign", [0, 1])
def test_conv_image_past_2_31(t, conv_big_inputs, misalign):
    """A 33-image batch of 256 x 256 x 1024 bytes (2.2 GB): the last image
    starts past 2**31.  misalign 0: the DMA form; 1: x one byte off 16-byte
    alignment, the byte-gather form.  Images 0 and 32 are the seeded inputs
    (the others repeat image 0); outputs of both are checked at sampled
    positions, borders included."""
    import oracle
    N, H, W, C, K, R, S = CONV_BIG
    pad, stride, dil = (1, 1), (1, 1), (1, 1)
    img_bytes = H * W * C
    assert (N - 1) * img_bytes >= BIG
    note(f"[case] conv large image N={N} H={H} W={W} C={C} K={K} misalign={misalign}")
    x0, xl, w = conv_big_inputs
    xb = torch.empty(N * img_bytes + 16, dtype=torch.int8, device="cuda")
    xv = xb[misalign:misalign + N * img_bytes].view(N, H, W, C)
    xv[0].copy_(torch.from_numpy(x0[0]))
    xv[1:N - 1].copy_(xv[0].unsqueeze(0).expand(N - 2, H, W, C))
    xv[N - 1].copy_(torch.from_numpy(xl[0]))
    wd = torch.from_numpy(w).cuda()
    P = t.conv2d_output_extent(H, R, pad[0], stride[0], dil[0])
    Q = t.conv2d_output_extent(W, S, pad[1], stride[1], dil[1])
    yb = torch.full((N * P * Q * K + 64,), SENT_C, dtype=torch.int32, device="cuda")
    st = t.conv2d_s8s8s32_nhwc(N, H, W, C, K, R, S, pad[0], pad[1], stride[0], stride[1], dil[0], dil[1],
                               xb.data_ptr() + misalign, wd.data_ptr(), yb.data_ptr(), 0)
    assert st == t.OK, t.tdi8_status_string(st)
    torch.cuda.synchronize()
    y = yb[:N * P * Q * K].view(N, P, Q, K)
    tail_ok = bool((yb[N * P * Q * K:] == SENT_C).all().item())
    rng = np.random.default_rng(22)
    ps = np.concatenate([[0, 0, P - 1, P - 1], rng.integers(0, P, 60)])
    qs = np.concatenate([[0, Q - 1, 0, Q - 1], rng.integers(0, Q, 60)])
    ks = rng.integers(0, K, ps.size)
    for n_dev, ximg in ((0, x0), (N - 1, xl), (N // 2, x0)):
        got = y[n_dev][torch.from_numpy(ps), torch.from_numpy(qs), torch.from_numpy(ks)].cpu().numpy()
        want = oracle.conv2d_points(ximg, w, np.zeros(ps.size, np.int64), ps, qs, ks, pad, stride, dil)
        assert np.array_equal(got, want), f"image {n_dev}: {int((got != want).sum())} mismatches"
    del xb, xv, yb, y
    torch.cuda.empty_cache()
    assert tail_ok, "output tail overwritten"
