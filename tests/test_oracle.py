"""Pins for the CPU oracle: brute force, a library special case, closed forms
and invariants.  Each pin is chosen so that a plausible slip in the oracle (a
dropped k term, a sign error, a transposed or mis-strided operand, a missing
wrap, a write into C's row padding) fails at least one of them."""
import itertools

import numpy as np
import pytest

import oracle
import synthetic

VALS = (-128, -1, 0, 1, 127)


def wrap32(x: int) -> int:
    x &= 0xFFFFFFFF
    return x - (1 << 32) if x >= (1 << 31) else x


def brute(A, B):
    """Pure-Python big-int triple loop on nested lists (logical A: MxK, B: KxN)."""
    M, K = len(A), len(A[0]) if A else 0
    N = len(B[0]) if B else 0
    return [[wrap32(sum(int(A[i][k]) * int(B[k][j]) for k in range(K))) for j in range(N)]
            for i in range(M)]


def run(A_log, B_log, b_col_major, lda_pad=0, ldb_pad=0):
    """Oracle on logical matrices stored with optional leading-dimension padding."""
    M, K = A_log.shape
    N = B_log.shape[1]
    A = np.full((M, K + lda_pad), 99, dtype=np.int8)
    A[:, :K] = A_log
    Bs = synthetic.store_b(B_log, b_col_major)
    B = np.full((Bs.shape[0], Bs.shape[1] + ldb_pad), -77, dtype=np.int8)
    B[:, :Bs.shape[1]] = Bs
    return oracle.gemm(A, B, b_col_major, M=M, N=N, K=K)


@pytest.mark.parametrize("b_col_major", [False, True])
def test_brute_force_all_small_value_combinations(b_col_major):
    # every A, B over the edge-value set for 1x1x1, 1x2x1, 2x1x1, 1x1x2, 2x1x2
    for (M, K, N) in [(1, 1, 1), (1, 2, 1), (2, 1, 1), (1, 1, 2), (2, 1, 2)]:
        for vals in itertools.product(VALS, repeat=M * K + K * N):
            A = np.array(vals[:M * K], dtype=np.int8).reshape(M, K)
            B = np.array(vals[M * K:], dtype=np.int8).reshape(K, N)
            assert run(A, B, b_col_major).tolist() == brute(A.tolist(), B.tolist())


@pytest.mark.parametrize("b_col_major", [False, True])
def test_brute_force_2x2x2_sampled_edge_values(b_col_major):
    rng = np.random.default_rng(7)
    for _ in range(3000):
        A = rng.choice(VALS, size=(2, 2)).astype(np.int8)
        B = rng.choice(VALS, size=(2, 2)).astype(np.int8)
        assert run(A, B, b_col_major).tolist() == brute(A.tolist(), B.tolist())


@pytest.mark.parametrize("b_col_major", [False, True])
def test_brute_force_random_shapes(b_col_major):
    rng = np.random.default_rng(11)
    for _ in range(200):
        M, N, K = (int(x) for x in rng.integers(1, [10, 8, 14]))
        A = rng.integers(-128, 128, size=(M, K)).astype(np.int8)
        B = rng.integers(-128, 128, size=(K, N)).astype(np.int8)
        pa, pb = (int(x) for x in rng.integers(0, 5, size=2))
        assert run(A, B, b_col_major, pa, pb).tolist() == brute(A.tolist(), B.tolist())


@pytest.mark.parametrize("b_col_major", [False, True])
def test_library_int64_matmul(b_col_major):
    rng = np.random.default_rng(3)
    for M, N, K in [(512, 512, 512), (37, 300, 129), (256, 1, 511), (1, 257, 64), (100, 100, 1)]:
        A = rng.integers(-128, 128, size=(M, K)).astype(np.int8)
        B = rng.integers(-128, 128, size=(K, N)).astype(np.int8)
        ref = (A.astype(np.int64) @ B.astype(np.int64)).astype(np.int32)  # exact, no wrap needed
        np.testing.assert_array_equal(run(A, B, b_col_major), ref)


@pytest.mark.parametrize("b_col_major", [False, True])
def test_closed_forms(b_col_major):
    for K in (1, 27, 64, 777):
        M, N = 5, 9
        ones_a, ones_b = np.ones((M, K), np.int8), np.ones((K, N), np.int8)
        assert (run(ones_a, ones_b, b_col_major) == K).all()
        lo_a, lo_b = np.full((M, K), -128, np.int8), np.full((K, N), -128, np.int8)
        assert (run(lo_a, lo_b, b_col_major) == 16384 * K).all()
        hi_a = np.full((M, K), 127, np.int8)
        assert (run(hi_a, lo_b, b_col_major) == -16256 * K).all()


def test_closed_form_at_large_k_and_wrap():
    # config-5 depth: |C| reaches 2**27 exactly
    K = 8192
    lo_a, lo_b = np.full((2, K), -128, np.int8), np.full((K, 3), -128, np.int8)
    C, ovf = oracle.gemm(lo_a, np.ascontiguousarray(lo_b.T), True, return_overflow=True)
    assert (C == 2 ** 27).all() and ovf == 0
    # past int32: 16384 * 131072 = 2**31 wraps to -2**31; one more term still wraps
    for K, expect in [(131071, 16384 * 131071), (131072, -(2 ** 31)), (131073, wrap32(16384 * 131073))]:
        a, b = np.full((1, K), -128, np.int8), np.full((1, K), -128, np.int8)
        C, ovf = oracle.gemm(a, b, True, return_overflow=True)
        assert int(C[0, 0]) == expect
        assert ovf == (0 if K == 131071 else 1)


@pytest.mark.parametrize("b_col_major", [False, True])
def test_identity_permutation_diagonal(b_col_major):
    rng = np.random.default_rng(5)
    K, N = 33, 17
    B = rng.integers(-128, 128, size=(K, N)).astype(np.int8)
    eye = np.eye(K, dtype=np.int8)
    np.testing.assert_array_equal(run(eye, B, b_col_major), B.astype(np.int32))
    perm = rng.permutation(K)
    P = eye[perm]
    np.testing.assert_array_equal(run(P, B, b_col_major), B[perm].astype(np.int32))
    d = rng.integers(-128, 128, size=K).astype(np.int8)
    D = np.diag(d).astype(np.int8)
    np.testing.assert_array_equal(run(D, B, b_col_major),
                                  d[:, None].astype(np.int32) * B.astype(np.int32))


def test_transpose_invariant_and_layout_equality():
    rng = np.random.default_rng(9)
    M, N, K = 23, 31, 45
    A = rng.integers(-128, 128, size=(M, K)).astype(np.int8)
    B = rng.integers(-128, 128, size=(K, N)).astype(np.int8)
    c_rr = run(A, B, False)
    c_rc = run(A, B, True)
    np.testing.assert_array_equal(c_rr, c_rc)
    # (AB)^T = B^T A^T : run the product of the transposes in both layouts
    for layout in (False, True):
        ct = run(np.ascontiguousarray(B.T), np.ascontiguousarray(A.T), layout)
        np.testing.assert_array_equal(ct.T, c_rr)


def test_k_additivity():
    rng = np.random.default_rng(13)
    M, N, K = 19, 21, 100
    A = rng.integers(-128, 128, size=(M, K)).astype(np.int8)
    B = rng.integers(-128, 128, size=(K, N)).astype(np.int8)
    full = run(A, B, True).astype(np.int64)
    for k1 in (1, 37, 64, 99):
        part = run(np.ascontiguousarray(A[:, :k1]), np.ascontiguousarray(B[:k1]), True).astype(np.int64) \
            + run(np.ascontiguousarray(A[:, k1:]), np.ascontiguousarray(B[k1:]), False).astype(np.int64)
        np.testing.assert_array_equal(full, part)


def test_freivalds_on_seeded_inputs():
    M, N, K = 300, 200, 513
    A, B = synthetic.gemm_inputs(M, N, K, seed=1)
    C = run(A, B, True).astype(np.int64)
    X = synthetic.freivalds_vectors(N, 8, seed=1)
    for x in X:
        np.testing.assert_array_equal(C @ x, A.astype(np.int64) @ (B.astype(np.int64) @ x))


def test_zero_k_and_padding_untouched():
    A = np.zeros((3, 4), np.int8)
    B = np.zeros((5, 4), np.int8)
    C = np.full((3, 7), 12345, np.int32)
    oracle.gemm(A, B, True, M=3, N=5, K=0, C=C)
    assert (C[:, :5] == 0).all() and (C[:, 5:] == 12345).all()
    # non-zero product: padding of ldc still untouched, window exact
    rng = np.random.default_rng(1)
    A = rng.integers(-128, 128, size=(3, 6)).astype(np.int8)
    B = rng.integers(-128, 128, size=(6, 5)).astype(np.int8)
    C = np.full((3, 9), -1, np.int32)
    oracle.gemm(A, B, False, M=3, N=5, K=6, C=C)
    assert C[:, :5].tolist() == brute(A.tolist(), B.tolist()) and (C[:, 5:] == -1).all()


def test_sampled_elements_match_full_product():
    M, N, K = 64, 48, 200
    A, B = synthetic.gemm_inputs(M, N, K, seed=2)
    for b_col_major in (False, True):
        Bs = synthetic.store_b(B, b_col_major)
        full = oracle.gemm(A, Bs, b_col_major)
        rows = np.arange(M * N) // N
        cols = np.arange(M * N) % N
        np.testing.assert_array_equal(oracle.gemm_elements(A, Bs, b_col_major, K, rows, cols),
                                      full.reshape(-1))
        assert oracle.gemm_element(A, Bs, b_col_major, K, 5, 7) == full[5, 7]


MUTANTS = {
    # a dropped k term in the column-major loop
    "drop_last_k_rc": ("for (int64_t k = 0; k < K; ++k) s +=", "for (int64_t k = 0; k < K - 1; ++k) s +="),
    # A read as unsigned bytes
    "unsigned_a": ("s += (int64_t)a[k] * (int64_t)b[k];", "s += (int64_t)(uint8_t)a[k] * (int64_t)b[k];"),
    # column-major B addressed with the wrong stride (transposed operand)
    "b_stride": ("const int8_t *b = B + j * ldb;", "const int8_t *b = B + j;"),
    # saturation instead of the two's-complement wrap
    "saturate": ("static int32_t wrap32(int64_t s) { return (int32_t)(uint32_t)(uint64_t)s; }",
                 "static int32_t wrap32(int64_t s) { return s > INT32_MAX ? INT32_MAX : s < INT32_MIN ? INT32_MIN : (int32_t)s; }"),
    # row-major B: a wrong sign on one operand
    "neg_rr": ("acc[j] += aik * (int64_t)b[j];", "acc[j] -= aik * (int64_t)b[j];"),
    # row-major B read with the column index and row index swapped
    "rr_swap": ("const int8_t *b = B + k * ldb;", "const int8_t *b = B + k;"),
}


def _pins_pass(lib) -> bool:
    """A compact run of the pins above against a candidate oracle library."""
    import ctypes
    f = lib.oracle_gemm_s8s8s32
    f.restype = ctypes.c_int64
    f.argtypes = [ctypes.c_int64] * 3 + [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                         ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_int64]

    def call(A, Bs, bcm, M, N, K):
        C = np.zeros((M, N), np.int32)
        f(M, N, K, A.ctypes.data, A.strides[0], Bs.ctypes.data, Bs.strides[0], bcm, C.ctypes.data, N)
        return C

    rng = np.random.default_rng(4)
    for _ in range(20):
        M, N, K = (int(x) for x in rng.integers(1, [10, 8, 14]))
        A = rng.integers(-128, 128, size=(M, K)).astype(np.int8)
        B = rng.integers(-128, 128, size=(K, N)).astype(np.int8)
        for bcm in (0, 1):
            Bs = synthetic.store_b(B, bool(bcm))
            if call(A, Bs, bcm, M, N, K).tolist() != brute(A.tolist(), B.tolist()):
                return False
    K = 131073
    a = np.full((1, K), -128, np.int8)
    if int(call(a, a.copy(), 1, 1, 1, K)[0, 0]) != wrap32(16384 * K):
        return False
    return True


def test_planted_mistakes_in_the_oracle_are_caught(tmp_path):
    """Each plausible slip, planted in a copy of oracle.c, fails the pins; the
    unmodified source passes the same check."""
    import ctypes
    import os
    import subprocess
    src = open(os.path.join(os.path.dirname(oracle.__file__), "oracle.c")).read()

    def build(text, name):
        c = tmp_path / (name + ".c")
        so = tmp_path / (name + ".so")
        c.write_text(text)
        subprocess.run(["gcc", "-O1", "-shared", "-fPIC", "-std=c11", "-o", str(so), str(c)], check=True)
        return ctypes.CDLL(str(so))

    assert _pins_pass(build(src, "unmodified"))
    for name, (old, new) in MUTANTS.items():
        assert src.count(old) == 1, name
        assert not _pins_pass(build(src.replace(old, new), name)), name
