"""Pins for the convolution oracle (oracle/oracle_conv.c), CPU only.

The oracle is the direct loop over the convolution's definition.  It is pinned
to things other than itself: SciPy's direct N-d correlation (a library
routine) on explicitly padded input and a dilated kernel, the reduction of a
1x1 convolution to the (separately pinned) matrix-product oracle, closed forms
(all ones counts the in-image taps; a centred delta filter returns the input;
an off-centre delta shifts it), additivity over channel groups, and planted
slips in copies of the C source that the pins must catch."""
import ctypes
import os
import subprocess

import numpy as np
import pytest

import oracle

scipy_signal = pytest.importorskip("scipy.signal")


def wrap32(v):
    return ((np.asarray(v, dtype=np.int64) + 2 ** 31) % 2 ** 32 - 2 ** 31).astype(np.int32)


def scipy_conv(x, w, pad, stride, dil):
    """SciPy's exact (direct-method) correlation over (h, w, c) per image and
    filter, on zero-padded input with the kernel's taps spread by dilation."""
    N, H, W, C = x.shape
    K, R, S, _ = w.shape
    (ph, pw), (sh, sw), (dh, dw) = pad, stride, dil
    xp = np.zeros((N, H + 2 * ph, W + 2 * pw, C), np.int64)
    xp[:, ph:ph + H, pw:pw + W, :] = x
    wd = np.zeros((K, dh * (R - 1) + 1, dw * (S - 1) + 1, C), np.int64)
    wd[:, ::dh, ::dw, :] = w
    outs = []
    for n in range(N):
        per_k = []
        for k in range(K):
            full = scipy_signal.correlate(xp[n], wd[k], mode="valid", method="direct")[:, :, 0]
            per_k.append(full[::sh, ::sw])
        outs.append(np.stack(per_k, axis=-1))
    return wrap32(np.stack(outs))


CASES = [  # (N, H, W, C, K, R, S, pad, stride, dil)
    (1, 5, 5, 3, 2, 3, 3, (1, 1), (1, 1), (1, 1)),
    (2, 7, 6, 4, 3, 3, 2, (0, 1), (2, 1), (1, 1)),
    (1, 9, 8, 2, 2, 3, 3, (2, 2), (1, 2), (2, 2)),
    (3, 4, 4, 5, 4, 1, 1, (0, 0), (1, 1), (1, 1)),
    (1, 6, 9, 3, 2, 2, 4, (1, 3), (3, 2), (1, 2)),
    (2, 3, 3, 16, 5, 3, 3, (1, 1), (1, 1), (1, 1)),
    (1, 8, 8, 1, 1, 5, 5, (2, 2), (2, 2), (1, 1)),
]


@pytest.mark.parametrize("case", CASES)
def test_matches_scipy_direct_correlation(case):
    N, H, W, C, K, R, S, pad, stride, dil = case
    rng = np.random.default_rng(sum(case[:7]))
    x = rng.integers(-128, 128, (N, H, W, C)).astype(np.int8)
    w = rng.integers(-128, 128, (K, R, S, C)).astype(np.int8)
    want = scipy_conv(x, w, pad, stride, dil)
    got = oracle.conv2d(x, w, pad, stride, dil)
    assert got.shape == want.shape and np.array_equal(got, want)


def test_extremes_against_scipy():
    x = np.full((1, 6, 6, 16), -128, np.int8)
    w = np.full((2, 3, 3, 16), -128, np.int8)
    assert np.array_equal(oracle.conv2d(x, w, (1, 1)), scipy_conv(x, w, (1, 1), (1, 1), (1, 1)))


def test_one_by_one_is_the_matrix_product():
    rng = np.random.default_rng(3)
    N, H, W, C, K = 2, 5, 7, 48, 9
    x = rng.integers(-128, 128, (N, H, W, C)).astype(np.int8)
    w = rng.integers(-128, 128, (K, 1, 1, C)).astype(np.int8)
    y = oracle.conv2d(x, w)
    g = oracle.gemm(x.reshape(N * H * W, C), w.reshape(K, C), True)
    assert np.array_equal(y.reshape(N * H * W, K), g)


@pytest.mark.parametrize("pad,stride,dil", [((1, 1), (1, 1), (1, 1)), ((2, 0), (2, 3), (1, 2)), ((0, 0), (1, 1), (3, 1))])
def test_all_ones_counts_in_image_taps(pad, stride, dil):
    N, H, W, C, K, R, S = 1, 7, 9, 5, 3, 3, 3
    x = np.ones((N, H, W, C), np.int8)
    w = np.ones((K, R, S, C), np.int8)
    y = oracle.conv2d(x, w, pad, stride, dil)
    P, Q = y.shape[1:3]
    for p in range(P):
        rows = sum(1 for r in range(R) if 0 <= p * stride[0] + r * dil[0] - pad[0] < H)
        for q in range(Q):
            cols = sum(1 for s in range(S) if 0 <= q * stride[1] + s * dil[1] - pad[1] < W)
            assert (y[0, p, q] == rows * cols * C).all()


def test_delta_filters_copy_and_shift():
    rng = np.random.default_rng(5)
    N, H, W, C = 2, 6, 5, 4
    x = rng.integers(-128, 128, (N, H, W, C)).astype(np.int8)
    # centred delta per channel (k = c), pad 1: the output is the input
    w = np.zeros((C, 3, 3, C), np.int8)
    for c in range(C):
        w[c, 1, 1, c] = 1
    assert np.array_equal(oracle.conv2d(x, w, (1, 1)), x.astype(np.int32))
    # delta at tap (0, 0) with pad 1: y[p][q] = x[p-1][q-1], zero on the first row/column
    w = np.zeros((C, 3, 3, C), np.int8)
    for c in range(C):
        w[c, 0, 0, c] = 1
    y = oracle.conv2d(x, w, (1, 1))
    assert (y[:, 0, :, :] == 0).all() and (y[:, :, 0, :] == 0).all()
    assert np.array_equal(y[:, 1:, 1:, :], x[:, :-1, :-1, :].astype(np.int32))


def test_additive_over_channel_groups():
    rng = np.random.default_rng(6)
    x = rng.integers(-128, 128, (2, 6, 6, 12)).astype(np.int8)
    w = rng.integers(-128, 128, (3, 3, 3, 12)).astype(np.int8)
    whole = oracle.conv2d(x, w, (1, 1), (2, 1))
    parts = [oracle.conv2d(np.ascontiguousarray(x[..., a:b]), np.ascontiguousarray(w[..., a:b]), (1, 1), (2, 1))
             for a, b in ((0, 5), (5, 12))]
    assert np.array_equal(whole, wrap32(parts[0].astype(np.int64) + parts[1]))


def test_points_match_full_output():
    rng = np.random.default_rng(7)
    x = rng.integers(-128, 128, (2, 9, 7, 16)).astype(np.int8)
    w = rng.integers(-128, 128, (5, 3, 3, 16)).astype(np.int8)
    y = oracle.conv2d(x, w, (1, 0), (2, 1), (1, 2))
    idx = [rng.integers(0, d, 200) for d in y.shape]
    assert np.array_equal(oracle.conv2d_points(x, w, *idx, pad=(1, 0), stride=(2, 1), dil=(1, 2)), y[tuple(idx)])


# ---- planted slips ---------------------------------------------------------------

CONV_MUTANTS = {
    "pad sign": ("p * stride_h + r * dil_h - pad_h", "p * stride_h + r * dil_h + pad_h"),
    "r and s swapped in the filter": ("w + ((k * R + r) * S + s) * C", "w + ((k * R + s) * S + r) * C"),
    "stride ignored along w": ("q * stride_w + s * dil_w - pad_w", "q + s * dil_w - pad_w"),
    "dilation ignored along h": ("p * stride_h + r * dil_h - pad_h", "p * stride_h + r - pad_h"),
    "border taps clamped instead of zero": (
        "const int64_t iw = q * stride_w + s * dil_w - pad_w;\n            if (iw < 0 || iw >= W) continue;",
        "int64_t iw = q * stride_w + s * dil_w - pad_w;\n            if (iw < 0) iw = 0; if (iw >= W) iw = W - 1;"),
    "unsigned input": ("sum += (int64_t)xp[c] * (int64_t)wp[c];", "sum += (int64_t)(uint8_t)xp[c] * (int64_t)wp[c];"),
}


def _conv_pins_pass(lib) -> bool:
    f = lib.oracle_conv2d_s8s8s32
    f.restype = ctypes.c_int64
    f.argtypes = [ctypes.c_int64] * 13 + [ctypes.c_void_p] * 3
    for case in CASES:
        N, H, W, C, K, R, S, pad, stride, dil = case
        rng = np.random.default_rng(sum(case[:7]))
        x = rng.integers(-128, 128, (N, H, W, C)).astype(np.int8)
        w = rng.integers(-128, 128, (K, R, S, C)).astype(np.int8)
        want = scipy_conv(x, w, pad, stride, dil)
        y = np.zeros(want.shape, np.int32)
        f(N, H, W, C, K, R, S, pad[0], pad[1], stride[0], stride[1], dil[0], dil[1],
          x.ctypes.data, w.ctypes.data, y.ctypes.data)
        if not np.array_equal(y, want):
            return False
    return True


def test_planted_mistakes_in_the_conv_oracle_are_caught(tmp_path):
    src = open(os.path.join(os.path.dirname(oracle.__file__), "oracle_conv.c")).read()

    def build(text, name):
        c = tmp_path / (name + ".c")
        so = tmp_path / (name + ".so")
        c.write_text(text)
        subprocess.run(["gcc", "-O1", "-fopenmp", "-shared", "-fPIC", "-std=c11", "-o", str(so), str(c)], check=True)
        return ctypes.CDLL(str(so))

    assert _conv_pins_pass(build(src, "unmodified"))
    for i, (name, (old, new)) in enumerate(CONV_MUTANTS.items()):
        assert src.count(old) >= 1, name
        assert not _conv_pins_pass(build(src.replace(old, new), f"m{i}")), f"mutant not caught: {name}"
