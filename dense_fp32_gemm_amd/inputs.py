"""Seeded synthetic operands for dense FP32 GEMM workloads.

This module holds no GEMM arithmetic.  It reproduces the two operand fills the
pages use, plus the seeded choice of output positions that large problems are
checked on, so that the GPU path and the oracle can be fed identical inputs.

* ``quarter_step`` -- the hash fill of the UIUC ECE408 Lecture 5 notes
  (tiled_matmul_basic.cu, host helper ``fillMatrix``): each value is an integer
  in {-3, ..., 4} times 0.25.  The page indexes a square matrix by its packed
  row-major index; a rows x cols matrix here uses the same packed index
  r*cols + c.  Every product and partial sum of such operands is exact in
  binary32 for K up to 2**20, which makes the product unique.
* ``uniform`` -- the linear congruential generator of the UIUC ECE408
  Lecture 12 final-project page (project_template.cu section 6, ``frand``):
  state <- 1664525*state + 1013904223 (mod 2**32), value = bits 8..31 of the
  state / 2**24 * 2 - 1, i.e. a multiple of 2**-23 in [-1, 1).  The page fills
  A first and then B from one stream seeded with 20250612.
* ``sample_positions`` -- the four corners of C, then (row, col) pairs drawn
  from the same generator seeded with 12345 (the seed of the page's sweep.cu).

The generator stream is computed with a jump-ahead (affine maps composed by
doubling) so that 10**8 values take seconds in numpy; ``tests/test_inputs.py``
pins it against the plain one-step recurrence.
"""
from __future__ import annotations

import numpy as np

UNIFORM_SEED = 20250612
SAMPLE_SEED = 12345
QUARTER_SEED_A = 1
QUARTER_SEED_B = 2

_MASK = 0xFFFFFFFF
_LCG_A = 1664525
_LCG_C = 1013904223
_CHUNK = 1 << 22


def _affine_pow(a: int, c: int, n: int) -> tuple[int, int]:
    """(a_n, c_n) such that n steps of s -> a*s + c equal s -> a_n*s + c_n."""
    ra, rc = 1, 0
    pa, pc = a, c
    while n:
        if n & 1:
            ra, rc = (pa * ra) & _MASK, (pa * rc + pc) & _MASK
        pa, pc = (pa * pa) & _MASK, (pa * pc + pc) & _MASK
        n >>= 1
    return ra, rc


class Lcg:
    """The 32-bit generator state <- 1664525*state + 1013904223 (mod 2**32)."""

    def __init__(self, seed: int):
        self.state = seed & _MASK

    def states(self, n: int) -> np.ndarray:
        """The next n states (uint32), advancing the generator by n steps."""
        out = np.empty(n, dtype=np.uint64)
        if n == 0:
            return out.astype(np.uint32)
        a1, c1 = _affine_pow(_LCG_A, _LCG_C, 1)
        out[0] = (a1 * self.state + c1) & _MASK
        filled = 1
        ja, jc = a1, c1          # map from state t to state t + filled
        while filled < n:
            m = min(filled, n - filled)
            # uint64 products wrap mod 2**64, which keeps the value mod 2**32.
            out[filled:filled + m] = (np.uint64(ja) * out[:m] + np.uint64(jc)) & np.uint64(_MASK)
            ja, jc = (ja * ja) & _MASK, (ja * jc + jc) & _MASK
            filled += m
        self.state = int(out[-1])
        return out.astype(np.uint32)


def _states_to_uniform(s: np.ndarray) -> np.ndarray:
    x = ((s >> np.uint32(8)) & np.uint32(0xFFFFFF)).astype(np.float32)
    return x / np.float32(16777216.0) * np.float32(2.0) - np.float32(1.0)


def uniform_fill(gen: Lcg, rows: int, cols: int) -> np.ndarray:
    """rows x cols float32 values in [-1, 1), row-major, drawn from ``gen``."""
    n = rows * cols
    out = np.empty(n, dtype=np.float32)
    for start in range(0, n, _CHUNK):
        m = min(_CHUNK, n - start)
        out[start:start + m] = _states_to_uniform(gen.states(m))
    return out.reshape(rows, cols)


def uniform(M: int, N: int, K: int, seed: int = UNIFORM_SEED):
    """(A, B) for C[M x N] = A[M x K] B[K x N]: A then B from one stream."""
    gen = Lcg(seed)
    A = uniform_fill(gen, M, K)
    B = uniform_fill(gen, K, N)
    return A, B


def quarter_step_fill(rows: int, cols: int, seed: int) -> np.ndarray:
    """rows x cols float32 values in {-0.75, ..., 1.00} from the hash fill."""
    n = rows * cols
    out = np.empty(n, dtype=np.float32)
    for start in range(0, n, _CHUNK):
        m = min(_CHUNK, n - start)
        idx = np.arange(start, start + m, dtype=np.uint64)
        x = (idx + np.uint64((seed * 7919) & _MASK)) & np.uint64(_MASK)
        x = (x * np.uint64(1103515245) + np.uint64(12345)) & np.uint64(_MASK)
        q = ((x >> np.uint64(16)) & np.uint64(7)).astype(np.int32) - 3
        out[start:start + m] = q.astype(np.float32) * np.float32(0.25)
    return out.reshape(rows, cols)


def quarter_step(M: int, N: int, K: int, seed_a: int = QUARTER_SEED_A,
                 seed_b: int = QUARTER_SEED_B):
    """(A, B) quarter-step operands; A uses seed 1 and B seed 2 by default."""
    return quarter_step_fill(M, K, seed_a), quarter_step_fill(K, N, seed_b)


def sample_positions(M: int, N: int, count: int = 4096, seed: int = SAMPLE_SEED):
    """(rows, cols) int64 arrays: the four corners, then seeded random pairs.

    Pair t takes two consecutive generator states s, s': row = (s >> 8) mod M
    and col = (s' >> 8) mod N.
    """
    if M <= 0 or N <= 0:
        return np.zeros(0, np.int64), np.zeros(0, np.int64)
    corners = [(0, 0), (0, N - 1), (M - 1, 0), (M - 1, N - 1)][:count]
    rest = count - len(corners)
    s = Lcg(seed).states(2 * rest).astype(np.int64) >> 8
    rows = np.concatenate([np.array([r for r, _ in corners], np.int64), s[0::2] % M])
    cols = np.concatenate([np.array([c for _, c in corners], np.int64), s[1::2] % N])
    return rows, cols
