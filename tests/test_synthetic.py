"""The seeded input generator: published SplitMix64 outputs, the counter form
against the sequential generator, the value range and layout independence."""
import os

import numpy as np

import synthetic

MASK = (1 << 64) - 1


def sequential_splitmix64(state: int, count: int):
    out = []
    for _ in range(count):
        state = (state + 0x9E3779B97F4A7C15) & MASK
        z = state
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & MASK
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & MASK
        out.append(z ^ (z >> 31))
    return out


def test_published_outputs_seed0():
    path = os.path.join(os.path.dirname(__file__), "golden", "splitmix64_seed0.txt")
    want = [int(line, 16) for line in open(path) if line.strip() and not line.startswith("#")]
    assert sequential_splitmix64(0, len(want)) == want
    got = synthetic.splitmix64_outputs(synthetic.stream_start(0, 0), 0, len(want))
    assert [int(x) for x in got] == want


def test_counter_form_equals_sequential_stream():
    for seed, tag in [(0, 1), (1, 2), (12345, 1), (2 ** 40 + 3, 2)]:
        s0 = synthetic.stream_start(seed, tag)
        seq = sequential_splitmix64(s0, 300)
        assert [int(x) for x in synthetic.splitmix64_outputs(s0, 0, 300)] == seq
        assert [int(x) for x in synthetic.splitmix64_outputs(s0, 100, 50)] == seq[100:150]


def test_matrix_values_are_low_bytes_in_row_major_order():
    A = synthetic.uniform_int8(7, 5, seed=3, tag=synthetic.TAG_A)
    seq = sequential_splitmix64(synthetic.stream_start(3, synthetic.TAG_A), 35)
    want = [((z & 0xFF) ^ 0x80) - 0x80 for z in seq]
    assert A.reshape(-1).tolist() == want
    assert A.dtype == np.int8 and A.flags.c_contiguous


def test_range_and_uniformity():
    v = synthetic.uniform_int8(1024, 1024, seed=0, tag=synthetic.TAG_B).reshape(-1)
    counts = np.bincount(v.view(np.uint8), minlength=256)
    assert (counts > 0).all() and v.min() == -128 and v.max() == 127
    expected = v.size / 256
    chi2 = float(((counts - expected) ** 2 / expected).sum())
    assert chi2 < 400  # 255 degrees of freedom; mean 255, sd ~22.6


def test_chunking_is_invisible():
    rows, cols = 3, (synthetic._CHUNK // 3) + 17   # spans two chunks
    A = synthetic.uniform_int8(rows, cols, seed=5, tag=1).reshape(-1)
    z = synthetic.splitmix64_outputs(synthetic.stream_start(5, 1), synthetic._CHUNK - 4, 8)
    tail = (z & np.uint64(0xFF)).astype(np.uint8).view(np.int8)
    assert (A[synthetic._CHUNK - 4:synthetic._CHUNK + 4] == tail).all()


def test_layouts_hold_the_same_logical_matrix():
    A, B = synthetic.gemm_inputs(6, 9, 4, seed=2)
    assert A.shape == (6, 4) and B.shape == (4, 9)
    Bc = synthetic.store_b(B, True)
    assert Bc.shape == (9, 4) and Bc.flags.c_contiguous and (Bc.T == B).all()
    assert (synthetic.store_b(B, False) == B).all()
    A2, B2 = synthetic.gemm_inputs(6, 9, 4, seed=3)
    assert not (A2 == A).all() and not (B2 == B).all()
    x = synthetic.freivalds_vectors(9, 4, seed=1)
    assert x.shape == (4, 9) and x.min() >= -8 and x.max() <= 7
