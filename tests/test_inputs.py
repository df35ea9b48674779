"""Pins of the seeded operand generators (CPU only).

The vectorised generators in dense_fp32_gemm_amd.inputs are checked against
the plain one-value-at-a-time recurrences they stand for (the Lecture 5 hash
fill and the Lecture 12 ``frand`` generator), written here as scalar Python
loops over Python integers.
"""
import numpy as np
import pytest

from dense_fp32_gemm_amd import inputs


def _frand_scalar(seed, n):
    """Lecture 12 project_template.cu section 6: one state update per value."""
    s = seed
    out = []
    for _ in range(n):
        s = (s * 1664525 + 1013904223) % 2**32
        x = (s >> 8) & 0xFFFFFF
        out.append(np.float32(np.float32(x) / np.float32(2**24) * np.float32(2.0) - np.float32(1.0)))
    return np.array(out, dtype=np.float32)


def _quarter_scalar(i, seed):
    """Lecture 5 tiled_matmul_basic.cu fillMatrix, for packed index i."""
    x = (i + seed * 7919) % 2**32
    x = (x * 1103515245 + 12345) % 2**32
    return np.float32((((x >> 16) & 7) - 3) * 0.25)


@pytest.mark.parametrize("n", [0, 1, 2, 3, 7, 64, 1000, 4097])
def test_lcg_matches_recurrence(n):
    got = inputs.uniform_fill(inputs.Lcg(inputs.UNIFORM_SEED), 1, n).ravel()
    ref = _frand_scalar(inputs.UNIFORM_SEED, n)
    assert got.tobytes() == ref.tobytes()


def test_uniform_is_one_stream_a_then_b():
    M, N, K = 5, 7, 3
    A, B = inputs.uniform(M, N, K)
    ref = _frand_scalar(inputs.UNIFORM_SEED, M * K + K * N)
    assert A.shape == (M, K) and B.shape == (K, N)
    assert A.ravel().tobytes() == ref[:M * K].tobytes()
    assert B.ravel().tobytes() == ref[M * K:].tobytes()


def test_chunking_does_not_change_the_stream(monkeypatch):
    ref_a, ref_b = inputs.uniform(13, 11, 9)
    qa = inputs.quarter_step_fill(13, 9, 1)
    monkeypatch.setattr(inputs, "_CHUNK", 5)
    a, b = inputs.uniform(13, 11, 9)
    assert a.tobytes() == ref_a.tobytes() and b.tobytes() == ref_b.tobytes()
    assert inputs.quarter_step_fill(13, 9, 1).tobytes() == qa.tobytes()


def test_uniform_value_set():
    A, B = inputs.uniform(64, 64, 64)
    v = np.concatenate([A.ravel(), B.ravel()]).astype(np.float64)
    assert v.min() >= -1.0 and v.max() < 1.0
    scaled = v * 2.0**23
    assert np.array_equal(scaled, np.round(scaled))   # multiples of 2**-23


@pytest.mark.parametrize("seed", [1, 2, 3, 4])
def test_quarter_step_matches_hash(seed):
    rows, cols = 9, 13
    got = inputs.quarter_step_fill(rows, cols, seed).ravel()
    ref = np.array([_quarter_scalar(i, seed) for i in range(rows * cols)], np.float32)
    assert got.tobytes() == ref.tobytes()
    assert set(np.unique(got * 4).astype(int)) <= set(range(-3, 5))


def test_quarter_step_large_index_wraps_like_uint32():
    # A 2048 x 2048 fill reaches index 4194303; check the tail against the hash.
    got = inputs.quarter_step_fill(2048, 2048, 2).ravel()[-5:]
    ref = [_quarter_scalar(2048 * 2048 - 5 + t, 2) for t in range(5)]
    assert got.tobytes() == np.array(ref, np.float32).tobytes()


def test_sample_positions():
    rows, cols = inputs.sample_positions(100, 37, count=4096)
    assert rows.shape == cols.shape == (4096,)
    assert list(zip(rows[:4], cols[:4])) == [(0, 0), (0, 36), (99, 0), (99, 36)]
    assert rows.min() >= 0 and rows.max() < 100 and cols.min() >= 0 and cols.max() < 37
    s = 12345
    for t in range(3):
        s = (s * 1664525 + 1013904223) % 2**32
        r = (s >> 8) % 100
        s = (s * 1664525 + 1013904223) % 2**32
        c = (s >> 8) % 37
        assert (rows[4 + t], cols[4 + t]) == (r, c)
    assert inputs.sample_positions(0, 5)[0].size == 0
