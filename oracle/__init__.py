"""CPU oracle for C = A x B with int8 inputs and int32 results.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything here.  The
product library never links, loads or calls it, and nothing here imports the
product package: the two share no code.

Contents
  * ``oracle.c`` (built with gcc into ``liboracle.so``): the plain triple loop
    over the definition C[i][j] = wrap32(sum_k A[i][k] * B[k][j]) with an exact
    int64 sum, for row-major A and row- or column-major B.
  * ``oracle_conv.c`` (same library): the direct 2-D convolution loop over its
    definition (NHWC input, KRSC weights, zero padding, stride, dilation).
  * ``selector.py``: the tile-configuration selection method of patent
    application CN114238853A (claims 1-6), written as plain Python from the
    claims' steps, with the readings of the steps whose formulas are missing
    from the text.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_SRCS = [_SRC, os.path.join(_HERE, "oracle_conv.c")]
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc (-O2, OpenMP).  Returns the library path."""
    if force or _stale():
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.run(["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-std=c11",
                        "-o", tmp, *_SRCS], check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _stale() -> bool:
    return not os.path.exists(_LIB) or any(os.path.getmtime(_LIB) < os.path.getmtime(f) for f in _SRCS)


def _load():
    global _lib
    if _lib is None:
        if _stale():
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        i64, p = ctypes.c_int64, ctypes.c_void_p
        lib.oracle_gemm_s8s8s32.restype = i64
        lib.oracle_gemm_s8s8s32.argtypes = [i64, i64, i64, p, i64, p, i64, ctypes.c_int, p, i64]
        lib.oracle_gemm_element.restype = ctypes.c_int32
        lib.oracle_gemm_element.argtypes = [i64, i64, i64, p, i64, p, i64, ctypes.c_int]
        lib.oracle_gemm_elements.restype = None
        lib.oracle_gemm_elements.argtypes = [i64, p, p, i64, p, i64, p, i64, ctypes.c_int, p]
        lib.oracle_num_threads.restype = ctypes.c_int
        lib.oracle_conv2d_s8s8s32.restype = i64
        lib.oracle_conv2d_s8s8s32.argtypes = [i64] * 13 + [p, p, p]
        lib.oracle_conv2d_points.restype = None
        lib.oracle_conv2d_points.argtypes = [i64, p, p, p, p] + [i64] * 11 + [p, p, p]
        lib.oracle_conv_out_extent.restype = i64
        lib.oracle_conv_out_extent.argtypes = [i64] * 5
        lib.oracle_set_num_threads.restype = None
        lib.oracle_set_num_threads.argtypes = [ctypes.c_int]
        _lib = lib
    return _lib


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def set_num_threads(n: int) -> None:
    """Threads used by the following calls (OpenMP)."""
    _load().oracle_set_num_threads(int(n))


def _check_storage(A, B, M, N, K, b_col_major):
    assert A.dtype == np.int8 and B.dtype == np.int8
    assert A.ndim == 2 and B.ndim == 2 and A.strides[1] == 1 and B.strides[1] == 1
    assert A.shape[0] >= M and A.shape[1] >= K
    if b_col_major:
        assert B.shape[0] >= N and B.shape[1] >= K
    else:
        assert B.shape[0] >= K and B.shape[1] >= N


def gemm(A: np.ndarray, B: np.ndarray, b_col_major: bool, M=None, N=None, K=None,
         C: np.ndarray | None = None, return_overflow: bool = False):
    """C = A x B from storage arrays.

    A: 2-D int8, row-major, shape (>=M, lda) with lda >= K (its row stride is lda).
    B: row-major K x N storage (b_col_major False) or N x K storage (True).
    Sizes default to the tight ones implied by the shapes.  Returns an (M, N)
    int32 array (or writes into C, whose rows may be padded).
    """
    if M is None:
        M = A.shape[0]
    if K is None:
        K = A.shape[1]
    if N is None:
        N = B.shape[0] if b_col_major else B.shape[1]
    _check_storage(A, B, M, N, K, b_col_major)
    if C is None:
        C = np.zeros((M, N), dtype=np.int32)
    assert C.dtype == np.int32 and C.strides[1] == 4 and C.shape[0] >= M and C.shape[1] >= N
    lda, ldb, ldc = A.strides[0], B.strides[0], C.strides[0] // 4
    ovf = _load().oracle_gemm_s8s8s32(M, N, K, A.ctypes.data, lda, B.ctypes.data, ldb,
                                      1 if b_col_major else 0, C.ctypes.data, ldc)
    return (C, int(ovf)) if return_overflow else C


def gemm_elements(A: np.ndarray, B: np.ndarray, b_col_major: bool, K: int,
                  rows: np.ndarray, cols: np.ndarray) -> np.ndarray:
    """C[rows[t], cols[t]] for each t, by the same definition."""
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    cols = np.ascontiguousarray(cols, dtype=np.int64)
    assert rows.shape == cols.shape
    out = np.empty(rows.shape, dtype=np.int32)
    _load().oracle_gemm_elements(rows.size, rows.ctypes.data, cols.ctypes.data, K,
                                 A.ctypes.data, A.strides[0], B.ctypes.data, B.strides[0],
                                 1 if b_col_major else 0, out.ctypes.data)
    return out


def gemm_element(A, B, b_col_major, K, i, j) -> int:
    return int(_load().oracle_gemm_element(i, j, K, A.ctypes.data, A.strides[0],
                                           B.ctypes.data, B.strides[0], 1 if b_col_major else 0))


# ---- convolution ---------------------------------------------------------------

def conv_out_extent(H: int, R: int, pad: int, stride: int, dil: int) -> int:
    return int(_load().oracle_conv_out_extent(H, R, pad, stride, dil))


def conv2d(x: np.ndarray, w: np.ndarray, pad=(0, 0), stride=(1, 1), dil=(1, 1), return_overflow=False):
    """y = conv2d(x, w): x int8 N x H x W x C (NHWC), w int8 K x R x S x C
    (KRSC); returns int32 N x P x Q x K (see oracle_conv.c)."""
    assert x.dtype == np.int8 and w.dtype == np.int8 and x.ndim == 4 and w.ndim == 4
    x = np.ascontiguousarray(x)
    w = np.ascontiguousarray(w)
    N, H, W, C = x.shape
    K, R, S, C2 = w.shape
    assert C == C2
    P = conv_out_extent(H, R, pad[0], stride[0], dil[0])
    Q = conv_out_extent(W, S, pad[1], stride[1], dil[1])
    y = np.zeros((N, P, Q, K), dtype=np.int32)
    ovf = _load().oracle_conv2d_s8s8s32(N, H, W, C, K, R, S, pad[0], pad[1], stride[0], stride[1],
                                         dil[0], dil[1], x.ctypes.data, w.ctypes.data, y.ctypes.data)
    return (y, int(ovf)) if return_overflow else y


def conv2d_points(x, w, n, p, q, k, pad=(0, 0), stride=(1, 1), dil=(1, 1)) -> np.ndarray:
    """y[n[t], p[t], q[t], k[t]] for each t, by the same definition."""
    x = np.ascontiguousarray(x)
    w = np.ascontiguousarray(w)
    _, H, W, C = x.shape
    _, R, S, _ = w.shape
    idx = [np.ascontiguousarray(v, dtype=np.int64) for v in (n, p, q, k)]
    out = np.empty(idx[0].shape, dtype=np.int32)
    _load().oracle_conv2d_points(idx[0].size, *(v.ctypes.data for v in idx), H, W, C, R, S,
                                 pad[0], pad[1], stride[0], stride[1], dil[0], dil[1],
                                 x.ctypes.data, w.ctypes.data, out.ctypes.data)
    return out
