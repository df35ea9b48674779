"""Pins of the CPU oracle (CPU only, no GPU).

The oracle (oracle/oracle.c) is the double-accumulating triple loop of the
UIUC ECE408 Lecture 12 final-project page (project_template.cu, section 3,
"CPU golden reference").  Nothing here compares the oracle with itself or
retypes its loop.  Each pin compares it with something the mathematics fixes:

* identity, permutation and all-ones matrices give exactly known products;
* rank-1 operands give one correctly rounded product per element;
* quarter-step operands (Lecture 5 hash fill) make every partial sum exact,
  so C equals an int64 matrix product divided by 16, bit for bit;
* uniform operands (Lecture 12 ``frand``) with K <= 128 have an exactly
  representable binary64 sum, so C is the correctly rounded exact sum,
  computed here with int64 arithmetic;
* every shape in {0..5}^3 against exact rational arithmetic (``fractions``)
  rounded once to binary32 by an independent round-to-nearest-even;
* a float64 library matmul (torch, CPU) agrees to within one ulp.

``test_planted_mistakes_fail_a_pin`` plants plausible mistakes in a copy of
oracle.c (dropped term, wrong sign, transposed operand, wrong index, float
accumulation, ...) and checks that each mutant fails at least one pin.
"""
import itertools
import os
import subprocess
import sys
from fractions import Fraction

import numpy as np
import pytest

import oracle
from dense_fp32_gemm_amd import inputs

ORC = oracle.load()


# ---------------------------------------------------------------------------
# Independent exact-value helpers
# ---------------------------------------------------------------------------
def bits(x):
    return np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)


def to_f32_rne(x: Fraction) -> np.float32:
    """Round an exact rational to the nearest binary32, ties to even.

    float(x) is the correctly rounded binary64; narrowing it can be off by at
    most one binary32 ulp, so the answer is one of three neighbours, chosen
    here by exact rational distance (ties: even significand).
    """
    f = np.float32(float(x))
    cands = [np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))]

    def key(c):
        return (abs(Fraction(float(c)) - x), int(np.float32(c).view(np.uint32)) & 1)
    return min(cands, key=key)


def exact_product_f32(A, B):
    """C rounded once from the exact rational product (tiny shapes only)."""
    M, K = A.shape
    N = B.shape[1]
    C = np.empty((M, N), np.float32)
    Af = [[Fraction(float(v)) for v in row] for row in A]
    Bf = [[Fraction(float(v)) for v in row] for row in B]
    for i in range(M):
        for j in range(N):
            s = sum((Af[i][k] * Bf[k][j] for k in range(K)), Fraction(0))
            C[i, j] = to_f32_rne(s)
    return C


def quarter_exact(A, B):
    """Quarter-step operands: C = ((4A) @ (4B)) / 16 in int64, exact in fp32."""
    ai = np.rint(A.astype(np.float64) * 4).astype(np.int64)
    bi = np.rint(B.astype(np.float64) * 4).astype(np.int64)
    assert np.array_equal(ai / 4, A) and np.array_equal(bi / 4, B)
    s = ai @ bi
    assert np.abs(s).max(initial=0) < 2**24 * 16
    return (s.astype(np.float64) / 16).astype(np.float32)


def uniform_exact_int(A):
    """frand values are multiples of 2**-23: return the int64 numerators."""
    ai = np.rint(A.astype(np.float64) * 2.0**23).astype(np.int64)
    assert np.array_equal(ai.astype(np.float64) / 2.0**23, A.astype(np.float64))
    return ai


def uniform_exact(A, B):
    """For K <= 128 the exact sum * 2**46 is an int64 below 2**53 in size, so
    it converts to binary64 exactly; one narrowing then rounds it correctly."""
    assert A.shape[1] <= 128
    s = uniform_exact_int(A) @ uniform_exact_int(B)
    return (s.astype(np.float64) * 2.0**-46).astype(np.float32)


# ---------------------------------------------------------------------------
# Pins on the real oracle
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("M,K", [(1, 1), (37, 53), (64, 64), (130, 17)])
def test_identity(M, K):
    A, _ = inputs.uniform(M, 1, K)
    assert np.array_equal(bits(ORC.gemm(A, np.eye(K, dtype=np.float32))), bits(A))
    assert np.array_equal(bits(ORC.gemm(np.eye(M, dtype=np.float32), A)), bits(A))


@pytest.mark.parametrize("n,m", [(1, 3), (9, 9), (31, 70), (65, 5)])
def test_permutation(n, m):
    rng = np.random.default_rng(n * 100 + m)
    perm = rng.permutation(n)
    P = np.zeros((n, n), np.float32)
    P[np.arange(n), perm] = 1.0                     # P[k, perm[k]] = 1
    X, _ = inputs.uniform(m, 1, n)                  # m x n
    # X @ P moves column k of X to column perm[k].
    want = np.empty_like(X)
    want[:, perm] = X
    assert np.array_equal(bits(ORC.gemm(X, P)), bits(want))
    # P @ Y moves row perm[k] of Y to row k.
    Y = np.ascontiguousarray(X.T)                   # n x m
    assert np.array_equal(bits(ORC.gemm(P, Y)), bits(Y[perm]))


@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (3, 5, 1000), (17, 33, 65), (8, 8, 4099)])
def test_all_ones(M, N, K):
    C = ORC.gemm(np.ones((M, K), np.float32), np.ones((K, N), np.float32))
    assert np.array_equal(C, np.full((M, N), K, np.float32))


@pytest.mark.parametrize("M,N", [(1, 1), (17, 33), (64, 100)])
def test_rank1_k1_is_one_rounding(M, N):
    A, B = inputs.uniform(M, N, 1)
    want = A.astype(np.float32) * B.astype(np.float32)     # IEEE binary32 product
    assert np.array_equal(bits(ORC.gemm(A, B)), bits(want))


@pytest.mark.parametrize("M,N,K", [(5, 7, 3), (33, 17, 1000)])
def test_rank1_quarter_step(M, N, K):
    u = inputs.quarter_step_fill(M, 1, 3)
    v = inputs.quarter_step_fill(1, N, 4)
    A = np.repeat(u, K, axis=1)
    B = np.repeat(v, K, axis=0)
    want = np.array([[Fraction(K) * Fraction(float(u[i, 0])) * Fraction(float(v[0, j]))
                      for j in range(N)] for i in range(M)], dtype=np.float64).astype(np.float32)
    assert np.array_equal(bits(ORC.gemm(A, B)), bits(want))


@pytest.mark.parametrize("M,N,K", [(512, 512, 512), (65, 77, 130), (1, 300, 2049)])
def test_quarter_step_exact(M, N, K):
    A, B = inputs.quarter_step(M, N, K)
    assert np.array_equal(bits(ORC.gemm(A, B)), bits(quarter_exact(A, B)))


@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (17, 33, 65), (64, 48, 128), (3, 200, 127)])
def test_uniform_small_k_exact(M, N, K):
    A, B = inputs.uniform(M, N, K)
    assert np.array_equal(bits(ORC.gemm(A, B)), bits(uniform_exact(A, B)))


def test_sampled_k128_exact_at_8192():
    """The 8192 x 8192 x 128 workload: samples are the correctly rounded sums."""
    M, N, K = 8192, 8192, 128
    A, B = inputs.uniform(M, N, K)
    r, c = inputs.sample_positions(M, N)
    ai, bi = uniform_exact_int(A), uniform_exact_int(B)
    s = np.einsum("tk,tk->t", ai[r], bi[:, c].T)
    want = (s.astype(np.float64) * 2.0**-46).astype(np.float32)
    assert np.array_equal(bits(ORC.gemm_at(A, B, r, c)), bits(want))


def test_brute_force_tiny_shapes():
    for M, N, K in itertools.product(range(6), repeat=3):
        for kind in ("uniform", "quarter"):
            if kind == "uniform":
                A, B = inputs.uniform(M, N, K, seed=1000 + 36 * M + 6 * N + K)
            else:
                A, B = inputs.quarter_step(M, N, K, 5 + M, 7 + N)
            want = exact_product_f32(A, B)
            got = ORC.gemm(A, B)
            assert got.shape == (M, N)
            assert np.array_equal(bits(got), bits(want)), (M, N, K, kind)
            if M and N:
                r, c = np.divmod(np.arange(M * N), N)
                assert np.array_equal(bits(ORC.gemm_at(A, B, r, c)), bits(want.ravel()))


@pytest.mark.parametrize("M,N,K", [(512, 512, 512), (1025, 1023, 1000), (17, 33, 65),
                                   (1, 1, 1), (200, 100, 3000)])
def test_float64_library_within_one_ulp(M, N, K):
    torch = pytest.importorskip("torch")
    A, B = inputs.uniform(M, N, K)
    ref = torch.matmul(torch.from_numpy(A).double(), torch.from_numpy(B).double()).float().numpy()
    got = ORC.gemm(A, B)
    d = np.abs(bits(got).astype(np.int64) - bits(ref).astype(np.int64))
    same_sign = np.signbit(got) == np.signbit(ref)
    assert np.all(same_sign | (got == 0) | (ref == 0))
    assert d.max() <= 1


def test_zero_k_gives_positive_zero():
    C = ORC.gemm(np.zeros((3, 0), np.float32), np.zeros((0, 4), np.float32))
    assert np.array_equal(bits(C), np.zeros((3, 4), np.uint32))


def test_empty_outputs():
    assert ORC.gemm(np.zeros((0, 5), np.float32), np.ones((5, 3), np.float32)).shape == (0, 3)
    assert ORC.gemm(np.ones((4, 5), np.float32), np.ones((5, 0), np.float32)).shape == (4, 0)


def test_leading_dimensions_and_padding():
    M, N, K = 19, 23, 31
    A, B = inputs.uniform(M, N, K)
    Ap = np.full((M, K + 5), np.nan, np.float32)
    Bp = np.full((K, N + 3), np.nan, np.float32)
    Cp = np.full((M + 2, N + 7), np.nan, np.float32)
    Ap[:, :K] = A
    Bp[:, :N] = B
    ORC.gemm(Ap[:, :K], Bp[:, :N], out=Cp[:M, :N])
    assert np.array_equal(bits(Cp[:M, :N]), bits(ORC.gemm(A, B)))
    assert np.isnan(Cp[:M, N:]).all() and np.isnan(Cp[M:]).all()


def test_gemm_at_equals_full_product():
    A, B = inputs.uniform(40, 30, 700)
    r, c = np.divmod(np.arange(40 * 30), 30)
    assert np.array_equal(bits(ORC.gemm_at(A, B, r, c)), bits(ORC.gemm(A, B).ravel()))


def test_thread_count_does_not_change_results():
    A, B = inputs.uniform(300, 200, 500)
    here = ORC.gemm(A, B)
    code = ("import sys, numpy as np; sys.path.insert(0, %r); import oracle; "
            "from dense_fp32_gemm_amd import inputs; A, B = inputs.uniform(300, 200, 500); "
            "sys.stdout.write(oracle.gemm(A, B).tobytes().hex())" % os.path.dirname(os.path.dirname(oracle.__file__)))
    env = dict(os.environ, OMP_NUM_THREADS="1")
    out = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True,
                         text=True, check=True).stdout
    assert bytes.fromhex(out) == here.tobytes()


def test_set_threads():
    A, B = inputs.uniform(97, 61, 300)
    before = ORC.threads()
    try:
        ORC.set_threads(1)
        assert ORC.threads() == 1
        one = ORC.gemm(A, B)
        ORC.set_threads(3)
        assert ORC.threads() == 3
        assert ORC.gemm(A, B).tobytes() == one.tobytes()
    finally:
        ORC.set_threads(before)
    assert ORC.threads() == before


# ---------------------------------------------------------------------------
# Planted mistakes: each mutant of oracle.c must fail at least one pin
# ---------------------------------------------------------------------------
def pin_failures(orc):
    """Runs square, packed pin cases (in bounds even for index mutants)."""
    failed = []

    def check(name, ok):
        if not ok:
            failed.append(name)

    n = 12
    A, B = inputs.uniform(n, n, n, seed=77)
    I = np.eye(n, dtype=np.float32)
    check("identity-right", np.array_equal(bits(orc.gemm(A, I)), bits(A)))
    check("identity-left", np.array_equal(bits(orc.gemm(I, A)), bits(A)))
    check("all-ones", np.array_equal(orc.gemm(np.ones((n, n), np.float32), np.ones((n, n), np.float32)),
                                     np.full((n, n), n, np.float32)))
    check("zero-k", np.array_equal(bits(orc.gemm(np.zeros((n, 0), np.float32), np.zeros((0, n), np.float32))),
                                   np.zeros((n, n), np.uint32)))
    for m in (16, 64):
        A, B = inputs.uniform(m, m, m, seed=m)
        want = uniform_exact(A, B)
        check(f"exact-rational-{m}", np.array_equal(bits(orc.gemm(A, B)), bits(want)))
        r, c = np.divmod(np.arange(m * m), m)
        check(f"exact-rational-at-{m}", np.array_equal(bits(orc.gemm_at(A, B, r, c)), bits(want.ravel())))
        Aq, Bq = inputs.quarter_step(m, m, m)
        check(f"quarter-{m}", np.array_equal(bits(orc.gemm(Aq, Bq)), bits(quarter_exact(Aq, Bq))))
        check(f"quarter-at-{m}", np.array_equal(bits(orc.gemm_at(Aq, Bq, r, c)),
                                                bits(quarter_exact(Aq, Bq).ravel())))
    return failed


MUTANTS = {
    "dropped-first-term": ("for (int k = 0; k < K; ++k) {", "for (int k = 1; k < K; ++k) {"),
    "dropped-last-term-at": ("for (int k = 0; k < K; ++k)\n            s +=",
                             "for (int k = 0; k < K - 1; ++k)\n            s +="),
    "wrong-sign": ("acc[j] += a * (double)brow[j];", "acc[j] -= a * (double)brow[j];"),
    "transposed-A": ("(double)A[(int64_t)i * lda + k]", "(double)A[(int64_t)k * lda + i]"),
    "transposed-B-at": ("(double)B[(int64_t)k * ldb + j]", "(double)B[(int64_t)j * ldb + k]"),
    "wrong-B-row": ("const float *brow = B + (int64_t)k * ldb;", "const float *brow = B + (int64_t)i * ldb;"),
    "float-accumulator": ("double *acc = (double *)malloc((size_t)N * sizeof(double));",
                          "float *acc = (float *)malloc((size_t)N * sizeof(float));"),
    "float-accumulator-at": ("double s = 0.0;", "float s = 0.0f;"),
    "reversed-output-index": ("C[(int64_t)i * ldc + j] = (float)acc[j];",
                              "C[(int64_t)i * ldc + j] = (float)acc[N - 1 - j];"),
    "swapped-sample-index": ("const int64_t i = rows[t];", "const int64_t i = cols[t];"),
    "nonzero-start": ("acc[j] = 0.0;", "acc[j] = 1e-30;"),
}


def test_real_oracle_passes_every_pin():
    assert pin_failures(ORC) == []


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistakes_fail_a_pin(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(oracle.SOURCE).read()
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    mutated = tmp_path / "oracle_mutant.c"
    mutated.write_text(src.replace(old, new))
    lib = oracle.build(str(mutated), str(tmp_path / "liboracle_mutant.so"))
    assert pin_failures(oracle.Oracle(lib)) != [], f"mutant {name} passed every pin"
