"""Parity of the implicit-GEMM convolution with the CPU convolution oracle,
through the C ABI.  Integer work: bit-exact on every compared output.  Small
shapes are compared in full for every general configuration; the layer shapes
timed by the bench are compared in full where the oracle is quick, else on
sampled outputs.  The output buffer carries a sentinel tail that must survive."""
import numpy as np
import pytest

import synthetic
from helpers import note

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

SENT = -123456789
TAIL = 64


@pytest.fixture(scope="module")
def t():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import tiled_dense_int8_amd as lib
    return lib


def run_conv(t, x, w, pad, stride, dil, config=None, seed_desc=""):
    """Device run; returns (y, sentinel tail intact)."""
    N, H, W, C = x.shape
    K, R, S, _ = w.shape
    P = t.conv2d_output_extent(H, R, pad[0], stride[0], dil[0])
    Q = t.conv2d_output_extent(W, S, pad[1], stride[1], dil[1])
    note(f"[case] conv N={N} H={H} W={W} C={C} K={K} R={R} S={S} pad={pad} stride={stride} dil={dil} "
         f"config={config} {seed_desc}")
    xd = torch.from_numpy(x).cuda()
    wd = torch.from_numpy(w).cuda()
    yb = torch.full((N * P * Q * K + TAIL,), SENT, dtype=torch.int32, device="cuda")
    args = (N, H, W, C, K, R, S, pad[0], pad[1], stride[0], stride[1], dil[0], dil[1],
            xd.data_ptr(), wd.data_ptr(), yb.data_ptr(), 0)
    st = t.conv2d_s8s8s32_nhwc(*args) if config is None else t.conv2d_s8s8s32_nhwc_with_config(config, *args)
    assert st == t.OK, t.tdi8_status_string(st)
    torch.cuda.synchronize()
    flat = yb.cpu().numpy()
    return flat[:N * P * Q * K].reshape(N, P, Q, K), bool((flat[N * P * Q * K:] == SENT).all())


def check(t, shape, pad=(0, 0), stride=(1, 1), dil=(1, 1), config=None, seed=0):
    import oracle
    N, H, W, C, K, R, S = shape
    x, w = synthetic.conv_inputs(N, H, W, C, K, R, S, seed)
    y, tail_ok = run_conv(t, x, w, pad, stride, dil, config, f"seed={seed}")
    want = oracle.conv2d(x, w, pad, stride, dil)
    assert y.shape == want.shape
    bad = int((y != want).sum())
    assert bad == 0, f"{bad} mismatches of {want.size}"
    assert tail_ok, "output tail overwritten"


SMALL = [  # (N, H, W, C, K, R, S), pad, stride, dil
    ((2, 9, 11, 16, 24, 3, 3), (1, 1), (1, 1), (1, 1)),
    ((1, 13, 7, 32, 70, 3, 3), (0, 2), (2, 1), (1, 1)),
    ((3, 8, 8, 48, 17, 1, 1), (0, 0), (1, 1), (1, 1)),
    ((1, 17, 15, 16, 130, 5, 3), (2, 1), (1, 2), (2, 1)),
    ((2, 6, 6, 64, 9, 7, 7), (3, 3), (1, 1), (1, 1)),
    ((1, 12, 12, 80, 33, 3, 3), (1, 1), (3, 3), (2, 2)),
]


@pytest.mark.parametrize("case", SMALL)
def test_every_general_config_small(t, case):
    shape, pad, stride, dil = case
    for cid in range(t.tile_config_count()):
        if t.tile_config_info(cid).family != 0:
            continue
        check(t, shape, pad, stride, dil, config=cid, seed=cid)


def test_selected_config_shapes(t):
    for (shape, pad, stride, dil) in SMALL:
        check(t, shape, pad, stride, dil)
    # few output pixels, long reduction (the contest's "C*R*S >> M, N" case)
    check(t, (1, 8, 8, 512, 32, 3, 3), (1, 1))
    # the whole image is padding for some taps: 1x1 input, 3x3 filter
    check(t, (4, 1, 1, 16, 8, 3, 3), (1, 1))


ODD = [  # channel counts that are not multiples of 16: the gather form
    ((2, 9, 11, 3, 24, 3, 3), (1, 1), (1, 1), (1, 1)),
    ((1, 13, 7, 1, 70, 3, 3), (0, 2), (2, 1), (1, 1)),
    ((3, 8, 8, 24, 17, 1, 1), (0, 0), (1, 1), (1, 1)),
    ((1, 17, 15, 5, 130, 5, 3), (2, 1), (1, 2), (2, 1)),
    ((2, 6, 6, 17, 9, 7, 7), (3, 3), (1, 1), (1, 1)),
    ((1, 12, 12, 8, 33, 3, 3), (1, 1), (3, 3), (2, 2)),
    # run form: filter rows of several 16-byte pieces, pieces that split a
    # tap's channels, padding wider than the image border, stride 2
    ((2, 15, 13, 3, 40, 7, 7), (3, 3), (2, 2), (1, 1)),
    ((1, 9, 10, 63, 20, 3, 3), (1, 1), (1, 1), (2, 1)),
    ((2, 5, 6, 7, 12, 5, 5), (4, 4), (1, 1), (1, 1)),
    ((1, 4, 21, 11, 8, 1, 9), (0, 4), (1, 3), (1, 1)),
]


@pytest.mark.parametrize("case", ODD)
def test_every_general_config_odd_channels(t, case):
    shape, pad, stride, dil = case
    for cid in range(t.tile_config_count()):
        if t.tile_config_info(cid).family != 0:
            continue
        check(t, shape, pad, stride, dil, config=cid, seed=cid + 100)


def test_first_layers(t):
    """Three input channels: the contest's 3 x 3 x 3 case (reduction 27) and
    a 7 x 7 stride-2 stem on a 224 x 224 image."""
    check(t, (2, 32, 32, 3, 64, 3, 3), (1, 1))
    check(t, (1, 224, 224, 3, 64, 7, 7), (3, 3), (2, 2))


def test_misaligned_operands_take_the_gather_form(t):
    """C a multiple of 16 but x and w off 16-byte alignment: same bytes as the
    oracle (and as the aligned DMA form)."""
    import oracle
    N, H, W, C, K, R, S = 2, 10, 9, 32, 40, 3, 3
    x, w = synthetic.conv_inputs(N, H, W, C, K, R, S, 7)
    P = t.conv2d_output_extent(H, R, 1, 1, 1)
    Q = t.conv2d_output_extent(W, S, 1, 1, 1)
    xb = torch.zeros(x.size + 64, dtype=torch.int8, device="cuda")
    wb = torch.zeros(w.size + 64, dtype=torch.int8, device="cuda")
    xb[1:1 + x.size].copy_(torch.from_numpy(x.reshape(-1)))
    wb[3:3 + w.size].copy_(torch.from_numpy(w.reshape(-1)))
    yb = torch.full((N * P * Q * K + TAIL,), SENT, dtype=torch.int32, device="cuda")
    note(f"[case] conv misaligned x+1 w+3 N={N} H={H} W={W} C={C} K={K}")
    assert t.conv2d_s8s8s32_nhwc(N, H, W, C, K, R, S, 1, 1, 1, 1, 1, 1, xb.data_ptr() + 1, wb.data_ptr() + 3,
                                 yb.data_ptr(), 0) == t.OK
    torch.cuda.synchronize()
    flat = yb.cpu().numpy()
    assert np.array_equal(flat[:N * P * Q * K].reshape(N, P, Q, K), oracle.conv2d(x, w, (1, 1), (1, 1), (1, 1)))
    assert (flat[N * P * Q * K:] == SENT).all()


def test_one_by_one_matches_the_gemm_entry(t):
    """A 1x1, stride-1 convolution is the product of the (N H W) x C image
    matrix with the K x C filter matrix (column-major B)."""
    N, H, W, C, K = 2, 16, 16, 64, 96
    x, w = synthetic.conv_inputs(N, H, W, C, K, 1, 1, 3)
    y, _ = run_conv(t, x, w, (0, 0), (1, 1), (1, 1))
    A = torch.from_numpy(x.reshape(N * H * W, C)).cuda()
    B = torch.from_numpy(w.reshape(K, C)).cuda()
    Cg = torch.empty((N * H * W, K), dtype=torch.int32, device="cuda")
    assert t.gemm_s8s8s32_bt(N * H * W, K, C, A.data_ptr(), C, B.data_ptr(), C, Cg.data_ptr(), K, 0) == t.OK
    torch.cuda.synchronize()
    assert np.array_equal(y.reshape(N * H * W, K), Cg.cpu().numpy())


def test_edge_cases(t):
    # C = 0: every output is 0
    x = np.zeros((2, 4, 4, 0), np.int8)
    w = np.zeros((5, 3, 3, 0), np.int8)
    y, tail_ok = run_conv(t, x, w, (1, 1), (1, 1), (1, 1))
    assert (y == 0).all() and tail_ok
    # no output position: the dilated filter is larger than the padded image
    xs, ws = synthetic.conv_inputs(1, 3, 3, 16, 4, 3, 3, 1)
    yb = torch.full((TAIL,), SENT, dtype=torch.int32, device="cuda")
    xd = torch.from_numpy(xs).cuda()
    wd = torch.from_numpy(ws).cuda()
    assert t.conv2d_output_extent(3, 3, 0, 1, 2) == 0
    assert t.conv2d_s8s8s32_nhwc(1, 3, 3, 16, 4, 3, 3, 0, 0, 1, 1, 2, 2, xd.data_ptr(), wd.data_ptr(),
                                 yb.data_ptr(), 0) == t.OK
    torch.cuda.synchronize()
    assert (yb.cpu().numpy() == SENT).all()
    # extremes: all -128, 3x3 with padding: interior outputs are 9 * C * 16384
    N, H, W, C, K = 1, 6, 6, 32, 8
    x = np.full((N, H, W, C), -128, np.int8)
    w = np.full((K, 3, 3, C), -128, np.int8)
    y, _ = run_conv(t, x, w, (1, 1), (1, 1), (1, 1))
    assert (y[:, 1:-1, 1:-1, :] == 9 * C * 16384).all() and (y[:, 0, 0, :] == 4 * C * 16384).all()


LAYERS = {  # the layer shapes the bench times (see bench.py)
    "conv3x3_56": ((32, 56, 56, 64, 64, 3, 3), (1, 1), (1, 1)),
    "conv3x3_14": ((32, 14, 14, 256, 256, 3, 3), (1, 1), (1, 1)),
    "conv1x1_28": ((32, 28, 28, 256, 512, 1, 1), (0, 0), (1, 1)),
    "conv3x3_s2": ((32, 56, 56, 128, 128, 3, 3), (1, 1), (2, 2)),
    "conv3x3_c3": ((32, 112, 112, 3, 64, 3, 3), (1, 1), (1, 1)),
}


@pytest.mark.parametrize("name", sorted(LAYERS))
def test_layer_shapes_sampled(t, name):
    import oracle
    shape, pad, stride = LAYERS[name]
    N, H, W, C, K, R, S = shape
    x, w = synthetic.conv_inputs(N, H, W, C, K, R, S, 0)
    y, tail_ok = run_conv(t, x, w, pad, stride, (1, 1))
    assert tail_ok
    rng = np.random.default_rng(1)
    n, p, q, k = (rng.integers(0, d, 4096) for d in y.shape)
    # plus the borders of the first image, where padding taps are zero
    P, Q = y.shape[1:3]
    bp = np.concatenate([np.zeros(Q, int), np.full(Q, P - 1), np.arange(P), np.arange(P)])
    bq = np.concatenate([np.arange(Q), np.arange(Q), np.zeros(P, int), np.full(P, Q - 1)])
    n = np.concatenate([n, np.zeros(bp.size, int)])
    k = np.concatenate([k, rng.integers(0, K, bp.size)])
    p = np.concatenate([p, bp])
    q = np.concatenate([q, bq])
    want = oracle.conv2d_points(x, w, n, p, q, k, pad=pad, stride=stride)
    assert np.array_equal(y[n, p, q, k], want)
    # the whole of image 0 against the full oracle
    full = oracle.conv2d(np.ascontiguousarray(x[:1]), w, pad, stride)
    assert np.array_equal(y[:1], full)


def test_graph_capture_and_stream(t):
    """The convolution entry only enqueues kernels: captured into a HIP graph,
    every replay reproduces the eager bytes (DMA form and byte-gather form),
    and a call on a side stream gives the same result."""
    for (shape, pad) in [((2, 9, 11, 16, 24, 3, 3), (1, 1)), ((2, 9, 11, 3, 24, 3, 3), (1, 1))]:
        N, H, W, C, K, R, S = shape
        note(f"[case] conv graph capture C={C}")
        x, w = synthetic.conv_inputs(N, H, W, C, K, R, S, 9)
        xd = torch.from_numpy(x).cuda()
        wd = torch.from_numpy(w).cuda()
        want = t.conv2d(xd, wd, pad)
        torch.cuda.synchronize()
        out = torch.empty_like(want)
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            t.conv2d(xd, wd, pad, out=out)
        s.synchronize()
        assert torch.equal(out, want)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            t.conv2d(xd, wd, pad, out=out)
        for r in range(3):
            out.fill_(-5)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(out, want), f"replay {r}"
            t.conv2d(xd, wd, pad)
            torch.cuda.synchronize()
