"""GPU parity: libgemm_f32.so (through its C ABI) against the CPU oracle.

Acceptance (tests/checks.py): bit-exact on quarter-step operands, where every
binary32 partial sum is exact and the product is unique; otherwise
|gpu - oracle| <= 1e-3 + 1e-3 * |oracle| per element.

Workloads: 512^3 quarter-step; the boundary set (1025,1023,1000), (1,1,1),
(17,33,65), (1000,1000,1000) on uniform[-1,1); 2048^3 uniform and
quarter-step (full oracle); 8192^3 and the rectangular sweep (8192,8192,128),
(16384,64,4096), (64,16384,4096), (4096,4096,16384) on uniform operands,
checked on 4096 seeded sample positions in the configuration the benchmark
times.  Small ragged shapes run on every kernel configuration.
"""
import functools
import sys

import numpy as np
import pytest

import oracle
from dense_fp32_gemm_amd import binding as gb
from dense_fp32_gemm_amd import inputs
from checks import assert_bit_exact, assert_close

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

CONFIGS = list(range(gb.gemm_f32_num_configs()))
CONFIG_IDS = [gb.gemm_f32_config_name(c) for c in CONFIGS]


def say(*msg):
    """Names the case before each GPU step (visible with pytest -s)."""
    print("[parity]", *msg, file=sys.__stderr__, flush=True)


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    say("device:", torch.cuda.get_device_name(0))
    return torch.device("cuda:0")


@functools.lru_cache(maxsize=4)
def operands(kind, M, N, K):
    if kind == "uniform":
        return inputs.uniform(M, N, K)
    return inputs.quarter_step(M, N, K)


def gpu_gemm(A, B, config=-1, dev=None, pad=(0, 0, 0), offset=(0, 0, 0), sentinel=np.nan):
    """Runs gemm_f32 on copies of A and B; returns (C window, full C buffer).

    pad adds columns to each operand's leading dimension; offset shifts each
    operand's base address by that many floats (4-byte aligned only).  The
    C buffer starts filled with `sentinel`.
    """
    M, K = A.shape
    N = B.shape[1]
    lda, ldb, ldc = max(1, K) + pad[0], max(1, N) + pad[1], max(1, N) + pad[2]
    dA = torch.full((offset[0] + M * lda + 1,), np.nan, dtype=torch.float32, device=dev)
    dB = torch.full((offset[1] + K * ldb + 1,), np.nan, dtype=torch.float32, device=dev)
    dC = torch.full((offset[2] + M * ldc + 1,), sentinel, dtype=torch.float32, device=dev)
    if M and K:
        dA[offset[0]:offset[0] + M * lda].view(M, lda)[:, :K].copy_(torch.from_numpy(A))
    if K and N:
        dB[offset[1]:offset[1] + K * ldb].view(K, ldb)[:, :N].copy_(torch.from_numpy(B))
    say(f"gemm_f32 config={config} M={M} N={N} K={K} ld=({lda},{ldb},{ldc}) off={offset}")
    rc = gb.gemm_f32_with_config(
        config, M, N, K,
        dA.data_ptr() + 4 * offset[0], lda,
        dB.data_ptr() + 4 * offset[1], ldb,
        dC.data_ptr() + 4 * offset[2], ldc,
        torch.cuda.current_stream().cuda_stream)
    assert rc == gb.GEMM_F32_OK, gb.gemm_f32_status_string(rc)
    torch.cuda.synchronize()
    full = dC.cpu().numpy()
    win = full[offset[2]:offset[2] + M * ldc].reshape(M, ldc)[:, :N] if M else np.zeros((0, N), np.float32)
    return np.ascontiguousarray(win), full


# ---------------------------------------------------------------------------
# The workloads
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("config", [-1] + CONFIGS, ids=["auto"] + CONFIG_IDS)
def test_512_quarter_step_bit_exact(dev, config):
    A, B = operands("quarter", 512, 512, 512)
    got, _ = gpu_gemm(A, B, config, dev)
    assert_bit_exact(got, oracle.gemm(A, B), f"512^3 quarter-step config {config}")


BOUNDARY = [(1025, 1023, 1000), (1, 1, 1), (17, 33, 65), (1000, 1000, 1000)]


@pytest.mark.parametrize("config", [-1] + CONFIGS, ids=["auto"] + CONFIG_IDS)
@pytest.mark.parametrize("shape", BOUNDARY, ids=lambda s: "x".join(map(str, s)))
def test_boundary_set_uniform(dev, shape, config):
    A, B = operands("uniform", *shape)
    got, _ = gpu_gemm(A, B, config, dev)
    assert_close(got, oracle.gemm(A, B), f"{shape} config {config}")


def test_2048_uniform_full(dev):
    A, B = operands("uniform", 2048, 2048, 2048)
    got, _ = gpu_gemm(A, B, -1, dev)
    assert_close(got, oracle.gemm(A, B), "2048^3 uniform")


def test_2048_quarter_step_bit_exact(dev):
    A, B = operands("quarter", 2048, 2048, 2048)
    got, _ = gpu_gemm(A, B, -1, dev)
    assert_bit_exact(got, oracle.gemm(A, B), "2048^3 quarter-step")


LARGE = [(8192, 8192, 8192), (8192, 8192, 128), (16384, 64, 4096),
         (64, 16384, 4096), (4096, 4096, 16384),
         # thin shapes where the rule keeps to 64-wide tiles
         (64, 32768, 4096), (65536, 64, 1024), (192, 16384, 4096),
         # a half-full second round: stream-K over the K-split tile
         (64, 24576, 4096)]


@pytest.mark.parametrize("shape", LARGE, ids=lambda s: "x".join(map(str, s)))
def test_large_sampled(dev, shape):
    M, N, K = shape
    A, B = inputs.uniform(M, N, K)
    got, _ = gpu_gemm(A, B, -1, dev, sentinel=np.nan)
    r, c = inputs.sample_positions(M, N)
    assert_close(got[r, c], oracle.gemm_at(A, B, r, c), f"{shape} sampled")
    # every element was written and is finite (the buffer started as NaN)
    assert np.isfinite(got).all()


# The scaling report's sizes (n = 128 ... 8192, doubling), each checked in
# full: all n^2 outputs of gemm_f32 on quarter-step operands against the
# oracle, bit for bit, with the configuration the report times.
REPORT_SIZES = [128 << i for i in range(7)]


@pytest.mark.parametrize("n", REPORT_SIZES)
def test_report_sizes_full_bit_exact(dev, n):
    from dense_fp32_gemm_amd import report
    A, B = inputs.quarter_step(n, n, n)
    dA = torch.from_numpy(A).to(dev)
    dB = torch.from_numpy(B).to(dev)
    dC = torch.full((n, n), float("nan"), dtype=torch.float32, device=dev)
    say(f"report size n={n}: gemm_f32 on quarter-step operands, full oracle")
    assert report._gemm(-1, dA, dB, dC, torch.cuda.current_stream()) == gb.GEMM_F32_OK
    torch.cuda.synchronize()
    got = dC.cpu().numpy()
    del dA, dB, dC
    assert_bit_exact(got, oracle.gemm(A, B), f"report size {n}")


# ---------------------------------------------------------------------------
# Every configuration on ragged shapes: several tiles plus a partial one in
# each dimension, K not a multiple of the panel depth.
# ---------------------------------------------------------------------------
RAGGED = [(300, 270, 77), (513, 385, 129), (97, 1100, 45), (1100, 70, 300), (33, 31, 2)]


@pytest.mark.parametrize("config", CONFIGS, ids=CONFIG_IDS)
@pytest.mark.parametrize("shape", RAGGED, ids=lambda s: "x".join(map(str, s)))
def test_ragged_bit_exact(dev, shape, config):
    A, B = operands("quarter", *shape)
    got, _ = gpu_gemm(A, B, config, dev)
    assert_bit_exact(got, oracle.gemm(A, B), f"{shape} config {config}")


# ---------------------------------------------------------------------------
# IEEE special values.  Whether an element of C is NaN, +Inf, -Inf or finite
# does not depend on the order of its sum: a NaN product (NaN, or Inf times
# zero) or +Inf meeting -Inf gives NaN, otherwise an infinite product decides
# the sign, and the finite operands here are too small to overflow.  So every
# configuration must classify each element of C exactly as the oracle does
# (and agree with it within tolerance where C is finite), including the
# elements fed by zero-filled or cleared padding.
# ---------------------------------------------------------------------------
SPECIAL_SHAPES = [(131, 97, 70), (300, 257, 1001)]


def special_operands(M, N, K, count=None):
    """Uniform operands with seeded NaN, +-Inf and +0 entries (about one in
    2000, or `count` per operand), and one forced Inf x 0 product."""
    A, B = (x.copy() for x in inputs.uniform(M, N, K))
    rng = np.random.default_rng(M * 1000003 + N * 1009 + K)
    specials = np.array([np.nan, np.inf, -np.inf, 0.0], dtype=np.float32)
    for X in (A, B):
        at = rng.choice(X.size, size=count or max(4, X.size // 2000), replace=False)
        X.flat[at] = rng.choice(specials, size=at.size)
    A[M // 2, K - 1] = np.inf
    B[K - 1, N // 3] = 0.0
    return A, B


@pytest.mark.parametrize("config", CONFIGS, ids=CONFIG_IDS)
@pytest.mark.parametrize("shape", SPECIAL_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_special_values_classified_as_the_oracle(dev, shape, config):
    M, N, K = shape
    A, B = special_operands(M, N, K)
    got, _ = gpu_gemm(A, B, config, dev)
    with np.errstate(invalid="ignore"):
        ref = oracle.gemm(A, B)
    kinds = {"nan": np.isnan, "+inf": np.isposinf, "-inf": np.isneginf}
    for name, f in kinds.items():
        bad = np.flatnonzero(f(got) != f(ref))
        assert bad.size == 0, f"{shape} config {config}: {bad.size} elements differ in being {name}; first {bad[0]}"
    assert all(f(ref).any() for f in kinds.values()), "the operands should produce every kind"
    fin = np.isfinite(ref)
    assert_close(got[fin], ref[fin], f"special {shape} finite part")


@pytest.mark.parametrize("config", CONFIGS, ids=CONFIG_IDS)
def test_permutation_pins_lane_layout(dev, config):
    """X @ P and P @ Y are exact permutations: any lane/register mix-up in
    operand or accumulator mapping moves a value to the wrong place."""
    n, m = 300, 260
    rng = np.random.default_rng(7)
    perm = rng.permutation(n)
    P = np.zeros((n, n), np.float32)
    P[np.arange(n), perm] = 1.0
    X, _ = inputs.uniform(m, 1, n)
    want = np.empty_like(X)
    want[:, perm] = X
    got, _ = gpu_gemm(X, P, config, dev)
    assert_bit_exact(got, want, "X @ P")
    Y = np.ascontiguousarray(X.T)
    got, _ = gpu_gemm(P, Y, config, dev)
    assert_bit_exact(got, Y[perm], "P @ Y")


@pytest.mark.parametrize("config", CONFIGS, ids=CONFIG_IDS)
def test_leading_dimensions_keep_padding(dev, config):
    M, N, K = 130, 200, 72
    A, B = operands("quarter", M, N, K)
    got, full = gpu_gemm(A, B, config, dev, pad=(3, 5, 7))
    assert_bit_exact(got, oracle.gemm(A, B), "padded ld")
    ldc = N + 7
    body = full[:M * ldc].reshape(M, ldc)
    assert np.isnan(body[:, N:]).all() and np.isnan(full[M * ldc:]).all()


@pytest.mark.parametrize("config", CONFIGS, ids=CONFIG_IDS)
def test_unaligned_bases(dev, config):
    """Bases 4-byte but not 16-byte aligned take the 32-bit load path."""
    M, N, K = 200, 160, 96
    A, B = operands("quarter", M, N, K)
    got, full = gpu_gemm(A, B, config, dev, offset=(1, 3, 2))
    assert_bit_exact(got, oracle.gemm(A, B), "offset bases")
    assert np.isnan(full[:2]).all()


WRITE_BACK = ["dma_64x64x32", "dma_64x128x32", "dma_128x64x32", "dma_64x64x32_sk",
              "dma_256x256x32_pipe", "dma_256x256x32_pipe_sk", "dma_128x128x64_pipe_lw2",
              "dma_128x128x64_pipe_lw2_sk", "dma_64x64x16_ksplit8_pipe",
              "dma_128x128x16_pipe", "dma_128x128x32_pipe"]


@functools.lru_cache(maxsize=1)
def write_back_case():
    M, N, K = 2049, 4097, 40          # M * N >= 2^23 elements
    A, B = operands("quarter", M, N, K)
    return A, B, oracle.gemm(A, B)


@pytest.mark.parametrize("name", ["auto"] + WRITE_BACK)
def test_write_back_c_stores_bit_exact_and_padding_kept(dev, name):
    """A large C whose rows are not 16-byte aligned runs the tiles'
    write-back twins (ordinary instead of streaming stores): bit-exact on
    quarter-step operands, and C's row padding (NaN) untouched."""
    config = -1 if name == "auto" else gb.config_names().index(name)
    A, B, want = write_back_case()
    M, K = A.shape
    N = B.shape[1]
    rc, text = gb.gemm_f32_describe(config, M, N, K, 4, K, 4, N, 4, N + 2)
    assert "c_store=write_back" in text, text
    got, full = gpu_gemm(A, B, config, dev, pad=(0, 0, 2))
    assert_bit_exact(got, want, f"{name} write-back C stores")
    body = full[:M * (N + 2)].reshape(M, N + 2)
    assert np.isnan(body[:, N:]).all() and np.isnan(full[M * (N + 2):]).all()


def test_k_zero_writes_positive_zero(dev):
    A = np.zeros((37, 0), np.float32)
    B = np.zeros((0, 45), np.float32)
    got, full = gpu_gemm(A, B, -1, dev, pad=(1, 0, 3))
    assert_bit_exact(got, np.zeros((37, 45), np.float32), "K=0")
    body = full[:37 * 48].reshape(37, 48)
    assert np.isnan(body[:, 45:]).all()


@pytest.mark.parametrize("M,N", [(0, 17), (17, 0)])
def test_empty_output_touches_nothing(dev, M, N):
    A, B = operands("uniform", M, N, 5)
    got, full = gpu_gemm(A, B, -1, dev)
    assert got.shape == (M, N) and np.isnan(full).all()


def test_transpose_invariant(dev):
    """(A B)^T = B^T A^T, bit-exact on quarter-step operands."""
    M, N, K = 384, 260, 200
    A, B = operands("quarter", M, N, K)
    C, _ = gpu_gemm(A, B, -1, dev)
    Ct, _ = gpu_gemm(np.ascontiguousarray(B.T), np.ascontiguousarray(A.T), -1, dev)
    assert_bit_exact(Ct.T, C, "transpose")


def test_all_ones_long_k(dev):
    K = 16384
    got, _ = gpu_gemm(np.ones((256, K), np.float32), np.ones((K, 256), np.float32), -1, dev)
    assert_bit_exact(got, np.full((256, 256), K, np.float32), "all-ones")


def test_identity_is_exact(dev):
    A, _ = operands("uniform", 1000, 1, 1000)
    got, _ = gpu_gemm(A, np.eye(1000, dtype=np.float32), -1, dev)
    assert_bit_exact(got, A, "A @ I")


def test_rank1_k1_is_one_rounding(dev):
    A, B = operands("uniform", 700, 900, 1)
    got, _ = gpu_gemm(A, B, -1, dev)
    assert_bit_exact(got, A * B, "K=1")


def test_runs_on_a_side_stream_and_repeats_bit_identically(dev):
    A, B = operands("uniform", 1000, 1000, 1000)
    dA = torch.from_numpy(A).to(dev)
    dB = torch.from_numpy(B).to(dev)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        c1 = gb.matmul(dA, dB)
        c2 = gb.matmul(dA, dB)
    s.synchronize()
    assert torch.equal(c1, c2)
    assert_close(c1.cpu().numpy(), oracle.gemm(A, B), "side stream")


def test_graph_capture_replays_match_eager(dev):
    """gemm_f32 enqueues plain kernel launches (no memset, no allocation), so
    it can be captured into a HIP graph; every replay must reproduce the
    eager result bit for bit (K = 0 included: its fill is a kernel too)."""
    A, B = operands("uniform", 1000, 1000, 1000)
    dA = torch.from_numpy(A).to(dev)
    dB = torch.from_numpy(B).to(dev)
    eager = gb.matmul(dA, dB)
    z = torch.empty((0, 64), dtype=torch.float32, device=dev)
    zb = torch.empty((64, 0), dtype=torch.float32, device=dev)
    out = torch.full((1000, 1000), float("nan"), device=dev)
    zout = torch.full((64, 64), float("nan"), device=dev)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        gb.matmul(dA, dB, out=out)          # warm-up on the capture stream
        gb.matmul(zb, z, out=zout)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph, stream=s):
        gb.matmul(dA, dB, out=out)
        gb.matmul(zb, z, out=zout)
    for _ in range(3):
        out.fill_(float("nan"))
        zout.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager)
        assert torch.equal(zout, torch.zeros_like(zout))


GRAPH_PLANS = [((2048, 2048, 512), "dma_128x128x64_pipe_lw2 "), ((4096, 4096, 128), "dma_128x128x16_pipe "),
               ((1025, 1023, 1000), "dma_64x64x16_ksplit8_pipe "), ((16384, 64, 4096), "dma_64x64x16_ksplit8_pipe "),
               ((512, 512, 512), "dma_32x32x32_ksplit8 "), ((640, 640, 2048), "dma_32x64x16_ksplit8 "),
               ((1000, 1000, 600), "dma_64x64x32_pipe_lw2_s4 "), ((2560, 2560, 2560), "dma_128x128x64_pipe_lw2_sk ")]


@pytest.mark.parametrize("shape,name", GRAPH_PLANS, ids=[n.strip() for _, n in GRAPH_PLANS])
def test_graph_capture_of_each_kernel_family(dev, shape, name):
    """The software-pipelined tiles (loader-wave ones and a stream-K plan
    with its clearing kernel included), the one-wave K-split tile and the
    remainder-strip kernel capture into a HIP graph like the rest: three
    replays, with eager work and synchronisations between them, each equal
    to the eager result bit for bit."""
    M, N, K = shape
    A, B = operands("uniform", M, N, K)
    dA = torch.from_numpy(A).to(dev)
    dB = torch.from_numpy(B).to(dev)
    rc, desc = gb.gemm_f32_describe(-1, M, N, K, dA.data_ptr(), K, dB.data_ptr(), N, dA.data_ptr(), N)
    assert rc == gb.GEMM_F32_OK and desc.startswith(name), desc
    say(f"graph capture {desc}")
    eager = gb.matmul(dA, dB)
    out = torch.full((M, N), float("nan"), device=dev)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        gb.matmul(dA, dB, out=out)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        gb.matmul(dA, dB, out=out)
    for _ in range(3):
        out.fill_(float("nan"))
        other = gb.matmul(dB[:64, :64].contiguous(), dA[:64, :64].contiguous())
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager)
        del other


def test_long_k_quarter_step_bit_exact(dev):
    """K = 2^20 - 16, the longest K for which quarter-step sums stay exact in
    binary32 (|partial sums| < 2^20 at 1/16 resolution), on the skinny path."""
    M, N, K = 64, 64, (1 << 20) - 16
    A, B = inputs.quarter_step(M, N, K)
    got, _ = gpu_gemm(A, B, -1, dev)
    assert_bit_exact(got, oracle.gemm(A, B), "long K")


def test_more_tiles_than_one_launch_holds(dev):
    """More than 2^20 output tiles: the grid is capped and each workgroup walks
    several tiles.  Checked on seeded samples plus the last rows (the tiles
    the second pass of the tile loop covers), gathered on the GPU."""
    M, N, K = 65536 + 64, 65536, 16
    cfg = gb.config_names().index("dma_64x64x32")
    A, B = inputs.uniform(M, N, K)
    dA = torch.from_numpy(A).to(dev)
    dB = torch.from_numpy(B).to(dev)
    dC = torch.full((M, N), float("nan"), dtype=torch.float32, device=dev)
    say(f"gemm_f32 config={cfg} M={M} N={N} K={K} (tile loop)")
    rc = gb.gemm_f32_with_config(cfg, M, N, K, dA.data_ptr(), K, dB.data_ptr(), N,
                                 dC.data_ptr(), N, torch.cuda.current_stream().cuda_stream)
    assert rc == gb.GEMM_F32_OK
    rc, desc = gb.gemm_f32_describe(cfg, M, N, K, dA.data_ptr(), K, dB.data_ptr(), N, dC.data_ptr(), N)
    assert "grid=1048576" in desc and "tiles=1025x1024" in desc, desc
    torch.cuda.synchronize()
    r, c = inputs.sample_positions(M, N)
    r = np.concatenate([r, np.full(64, M - 1), np.arange(M - 64, M)])
    c = np.concatenate([c, np.arange(0, N, N // 64), np.full(64, N - 1)])
    got = dC[torch.from_numpy(r).to(dev), torch.from_numpy(c).to(dev)].cpu().numpy()
    assert_close(got, oracle.gemm_at(A, B, r, c), "tile loop samples")
    assert bool(torch.isfinite(dC).all())
    del dC


def test_random_shapes_layouts_and_configs(dev):
    """Seeded fuzz: random small shapes, leading-dimension padding and base
    offsets, each on a random configuration, bit-exact on quarter-step."""
    rng = np.random.default_rng(20250612)
    for trial in range(40):
        M, N, K = (int(x) for x in rng.integers(1, 300, size=3))
        config = int(rng.integers(-1, gb.gemm_f32_num_configs()))
        pad = tuple(int(x) for x in rng.integers(0, 9, size=3))
        off = tuple(int(x) for x in rng.integers(0, 4, size=3))
        A, B = inputs.quarter_step(M, N, K, 11 + trial, 13 + trial)
        got, _ = gpu_gemm(A, B, config, dev, pad=pad, offset=off)
        assert_bit_exact(got, oracle.gemm(A, B), f"trial {trial}: {(M, N, K)} config {config} pad {pad} off {off}")


# ---------------------------------------------------------------------------
# The shape rule's branches, one shape each, through the automatic plan
# (config -1): the plan is the expected one and its C is the oracle's, bit
# for bit, on quarter-step operands, with C's row padding untouched.
# ---------------------------------------------------------------------------
RULE_BRANCHES = [((535, 1913, 700), "dma_32x64x16_ksplit8 "),         # two rounds of 32 x 64
                 ((1913, 535, 700), "dma_64x32x16_ksplit8 "),         # two rounds of 64 x 32
                 ((660, 1684, 979), "dma_32x32x32_ksplit4 "),         # just past one round, K < 1150
                 ((1100, 1100, 1100), "dma_64x64x16_ksplit8_pipe_sk "),
                 ((1197, 2414, 2200), "dma_64x64x16_ksplit8_pipe "),  # three fuller rounds
                 ((2282, 1391, 771), "dma_128x128x32_pipe "),         # one round of 128 x 128, 32-deep
                 ((3394, 1064, 960), "dma_128x128x64_pipe_lw2 "),     # the same, 64-deep
                 ((3428, 2297, 1100), "dma_128x128x32_pipe "),        # a nearly full second round
                 ((1025, 1025, 2000), "dma_64x64x16_ksplit8_pipe ")]  # row and column strips


@pytest.mark.parametrize("shape,name", RULE_BRANCHES, ids=["x".join(map(str, s)) for s, _ in RULE_BRANCHES])
def test_rule_branches_bit_exact(dev, shape, name):
    M, N, K = shape
    rc, desc = gb.gemm_f32_describe(-1, M, N, K, 16, K, 16, N, 16, N + 3)
    assert rc == gb.GEMM_F32_OK and desc.startswith(name), desc
    A, B = operands("quarter", M, N, K)
    got, full = gpu_gemm(A, B, -1, dev, pad=(0, 0, 3))
    assert_bit_exact(got, oracle.gemm(A, B), f"{shape} {desc}")
    body = full[:M * (N + 3)].reshape(M, N + 3)
    assert np.isnan(body[:, N:]).all() and np.isnan(full[M * (N + 3):]).all()


# ---------------------------------------------------------------------------
# Stream-K: more tiles than compute units, so the K-panels of some tiles are
# split between two workgroups that add their partial sums into C.
# ---------------------------------------------------------------------------
STREAMK = [("dma_64x64x16_ksplit8_pipe_sk", (1025, 1023, 1000)),
           ("dma_64x64x32_ksplit4_sk", (1025, 1023, 1000)), ("dma_64x64x32_sk", (1100, 1050, 77)),
           ("dma_64x64x64_sk", (1100, 1050, 200)),
           ("dma_64x64x64_sk", (1025, 1023, 1000)),
           # pieces of 1-5 K-panels for 8 groups (K = 77); a ragged K over two
           # and three rounds of tiles
           ("dma_64x64x16_ksplit8_pipe_sk", (1100, 1050, 77)), ("dma_64x64x16_ksplit8_pipe_sk", (1300, 1300, 1003)),
           ("dma_64x64x16_ksplit8_pipe_sk", (2000, 700, 4100)),
           # ranges of about 2.9 and 3.4 tiles: two or three whole tiles
           # before each workgroup's start and end pieces
           ("dma_64x64x16_ksplit8_pipe_sk", (1252, 2307, 600)), ("dma_128x128x64_pipe_lw2_sk", (4500, 3000, 520)),
           ("dma_128x128x32_w16_sk", (2176, 2100, 1000)), ("dma_128x128x64_pipe_lw2_sk", (2176, 2100, 1003)),
           ("dma_256x256x32_pipe_sk", (4352, 4200, 203)), ("dma_256x256x32_pipe_sk", (4352, 4200, 200))]


@pytest.mark.parametrize("name,shape", STREAMK, ids=[f"{n}-{'x'.join(map(str, s))}" for n, s in STREAMK])
def test_streamk_bit_exact_and_padding_kept(dev, name, shape):
    M, N, K = shape
    cfg = gb.config_names().index(name)
    rc, desc = gb.gemm_f32_describe(cfg, M, N, K, 16, K, 16, N, 16, N + 5)
    assert rc == gb.GEMM_F32_OK and "grid=256 " in desc, desc
    A, B = operands("quarter", M, N, K)
    got, full = gpu_gemm(A, B, cfg, dev, pad=(0, 0, 5))
    assert_bit_exact(got, oracle.gemm(A, B), f"{shape} {name}")
    body = full[:M * (N + 5)].reshape(M, N + 5)
    assert np.isnan(body[:, N:]).all() and np.isnan(full[M * (N + 5):]).all()


@pytest.mark.parametrize("name,shape", STREAMK[:4], ids=[f"{n}-{'x'.join(map(str, s))}" for n, s in STREAMK[:4]])
def test_streamk_uniform_within_tolerance_and_deterministic(dev, name, shape):
    """Each shared tile receives exactly two partial sums added to +0.0, and
    binary32 addition is commutative, so the result does not depend on which
    workgroup finishes first: repeated calls agree bit for bit."""
    cfg = gb.config_names().index(name)
    A, B = operands("uniform", *shape)
    first, _ = gpu_gemm(A, B, cfg, dev)
    assert_close(first, oracle.gemm(A, B), f"{shape} {name}")
    for _ in range(3):
        again, _ = gpu_gemm(A, B, cfg, dev)
        assert_bit_exact(again, first, f"{shape} {name} repeat")


@pytest.mark.parametrize("config", [c for c in CONFIGS if gb.gemm_f32_config_name(c).startswith("dma")],
                         ids=[n for n in CONFIG_IDS if n.startswith("dma")])
def test_b_chunks_crossing_column_n_leave_c_clean(dev, config):
    """N % 4 != 0 with NaN in B's row padding: 128-bit B loads that run past
    column N pick up NaN (or the next row) in LDS columns >= N, which must
    not reach any stored element; K % 4 == 0 with NaN in A's padding, and
    unaligned bases, exercise 128-bit A loads from 4-byte aligned rows."""
    M, N, K = 130, 270, 72
    A, B = operands("quarter", M, N, K)
    for pad, off in (((0, 0, 0), (0, 0, 0)), ((1, 3, 2), (0, 0, 0)), ((3, 1, 0), (1, 2, 3))):
        got, full = gpu_gemm(A, B, config, dev, pad=pad, offset=off)
        assert_bit_exact(got, oracle.gemm(A, B), f"pad {pad} off {off}")
        ldc = N + pad[2]
        body = full[off[2]:off[2] + M * ldc].reshape(M, ldc)
        assert np.isnan(body[:, N:]).all() and np.isnan(full[off[2] + M * ldc:]).all()


@pytest.mark.parametrize("shape,expect", [((1100, 1100, 1100), "dma_64x64x16_ksplit8_pipe_sk "),
                                          ((574, 1850, 1256), "dma_64x64x32_ksplit4_sk ")])
def test_streamk_in_graph_and_on_concurrent_streams(dev, shape, expect):
    """The stream-K plan is two kernels (clear the shared tiles, then the
    workers' atomic adds) and no memset: it captures into a HIP graph whose
    replays reproduce the eager result bit for bit, and two calls running at
    once on different streams share nothing."""
    M, N, K = shape
    A, B = operands("uniform", M, N, K)
    dA = torch.from_numpy(A).to(dev)
    dB = torch.from_numpy(B).to(dev)
    rc, desc = gb.gemm_f32_describe(-1, M, N, K, dA.data_ptr(), K, dB.data_ptr(), N, dA.data_ptr(), N)
    assert desc.startswith(expect), desc
    say(f"stream-K eager, graph and concurrent streams, {M}x{N}x{K}")
    eager = gb.matmul(dA, dB)
    torch.cuda.synchronize()
    assert_close(eager.cpu().numpy(), oracle.gemm(A, B), "stream-K eager")
    out = torch.full((M, N), float("nan"), device=dev)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        gb.matmul(dA, dB, out=out)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        gb.matmul(dA, dB, out=out)
    for _ in range(3):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager)
    streams = [torch.cuda.Stream() for _ in range(2)]
    outs = [torch.full((M, N), float("nan"), device=dev) for _ in range(2)]
    torch.cuda.synchronize()
    for _ in range(4):
        for st, o in zip(streams, outs):
            with torch.cuda.stream(st):
                gb.matmul(dA, dB, out=o)
    torch.cuda.synchronize()
    for o in outs:
        assert torch.equal(o, eager)


# ---------------------------------------------------------------------------
# Remainder strips: 1-4 rows (columns) past one round of K-split tiles,
# computed with FMAs, spread over all the tiles' workgroups.
# ---------------------------------------------------------------------------
STRIP = [((1025, 1023, 1000), "strip_rows=1"), ((1028, 1000, 1000), "strip_rows=4"),
         ((1026, 1001, 1001), "strip_rows=2"), ((1027, 1024, 1300), "strip_rows=3"),
         ((1023, 1025, 1000), "strip_cols=1"), ((1000, 1028, 1000), "strip_cols=4"),
         ((1001, 1026, 1001), "strip_cols=2"), ((1024, 1027, 1300), "strip_cols=3"),
         # the strip's shortest and longest K (rows x K up to 4096)
         ((1025, 1023, 513), "strip_rows=1"), ((1025, 1023, 2047), "strip_rows=1"),
         ((1023, 1025, 2047), "strip_cols=1"), ((1025, 1023, 4096), "strip_rows=1"),
         ((1023, 1025, 4096), "strip_cols=1"), ((1026, 1023, 2048), "strip_rows=2"),
         ((1025, 1000, 2500), "strip_rows=1"),
         # a row and a column strip (the corner in the row strip), K up to 3072
         ((1025, 1025, 1000), "strip_rows=1 strip_cols=1"), ((1028, 1025, 1000), "strip_rows=4 strip_cols=1"),
         ((1025, 1026, 2048), "strip_rows=1 strip_cols=2"), ((1027, 1027, 1300), "strip_rows=3 strip_cols=3"),
         ((1026, 1028, 1024), "strip_rows=2 strip_cols=4"), ((1025, 1025, 3000), "strip_rows=1 strip_cols=1"),
         # K from 257 on
         ((1028, 1000, 400), "strip_rows=4"), ((1023, 1026, 257), "strip_cols=2"),
         ((1025, 1025, 300), "strip_rows=1 strip_cols=1")]


@pytest.mark.parametrize("shape,strip", STRIP, ids=["x".join(map(str, s)) for s, _ in STRIP])
def test_strips_bit_exact_and_padding_kept(dev, shape, strip):
    M, N, K = shape
    rc, desc = gb.gemm_f32_describe(-1, M, N, K, 16, K + 3, 16, N + 1, 16, N + 5)
    assert rc == gb.GEMM_F32_OK and desc.replace(" lds=poisoned", "").endswith(" " + strip), desc
    A, B = operands("quarter", M, N, K)
    got, full = gpu_gemm(A, B, -1, dev, pad=(3, 1, 5))
    assert_bit_exact(got, oracle.gemm(A, B), f"{shape} strip")
    body = full[:M * (N + 5)].reshape(M, N + 5)
    assert np.isnan(body[:, N:]).all() and np.isnan(full[M * (N + 5):]).all()


# A remainder of 5-7 rows or columns with K just past 512: once planned as a
# strip wider than the strip kernel sums (fixed), now a plain plan.
WIDE_REMAINDER = [(1029, 1000, 600), (1030, 1000, 600), (1031, 1000, 513), (1000, 1031, 513)]


@pytest.mark.parametrize("shape", WIDE_REMAINDER, ids=lambda s: "x".join(map(str, s)))
def test_wide_remainders_bit_exact_and_padding_kept(dev, shape):
    M, N, K = shape
    rc, desc = gb.gemm_f32_describe(-1, M, N, K, 16, K, 16, N, 16, N + 3)
    assert rc == gb.GEMM_F32_OK and "strip" not in desc, desc
    A, B = operands("quarter", M, N, K)
    got, full = gpu_gemm(A, B, -1, dev, pad=(0, 0, 3))
    assert_bit_exact(got, oracle.gemm(A, B), f"{shape}")
    body = full[:M * (N + 3)].reshape(M, N + 3)
    assert np.isnan(body[:, N:]).all() and np.isnan(full[M * (N + 3):]).all()


@pytest.mark.parametrize("shape", [(1025, 1023, 1000), (1023, 1025, 1000)], ids=["rows", "cols"])
def test_strips_special_values_classified_as_the_oracle(dev, shape):
    """NaN and +-Inf in the strip's rows (columns) of A (B) and elsewhere:
    every element of C, strip included, is NaN, +Inf, -Inf or finite exactly
    when the oracle's is (the classification does not depend on summation
    order), and finite elements are within tolerance."""
    M, N, K = shape
    A, B = special_operands(M, N, K)
    A[M - 1, 7] = np.inf          # the strip row (or, for columns, a row the strip spans)
    B[11, N - 1] = -np.inf        # the strip column (or a column the row strip spans)
    got, _ = gpu_gemm(A, B, -1, dev)
    with np.errstate(invalid="ignore"):
        ref = oracle.gemm(A, B)
    for name, f in {"nan": np.isnan, "+inf": np.isposinf, "-inf": np.isneginf}.items():
        bad = np.flatnonzero(f(got) != f(ref))
        assert bad.size == 0, f"{shape}: {bad.size} elements differ in being {name}; first {bad[0]}"
    fin = np.isfinite(ref)
    assert np.isfinite(ref[M - 1]).sum() < N or np.isfinite(ref[:, N - 1]).sum() < M
    assert_close(got[fin], ref[fin], f"strip special {shape} finite part")


@pytest.mark.parametrize("shape", [(1026, 1001, 1001), (1001, 1026, 1001)], ids=["rows", "cols"])
def test_strips_uniform_within_tolerance_and_deterministic(dev, shape):
    A, B = operands("uniform", *shape)
    first, _ = gpu_gemm(A, B, -1, dev)
    assert_close(first, oracle.gemm(A, B), f"strip uniform {shape}")
    for _ in range(2):
        again, _ = gpu_gemm(A, B, -1, dev)
        assert_bit_exact(again, first, f"strip repeat {shape}")


# ---------------------------------------------------------------------------
# Split-K through a caller's workspace (few tiles, long K).
# ---------------------------------------------------------------------------
def gpu_gemm_ws(A, B, dev, ws_bytes=None, ldc_pad=0):
    M, K = A.shape
    N = B.shape[1]
    need = gb.gemm_f32_ws_size(M, N, K)
    ws_bytes = need if ws_bytes is None else ws_bytes
    dA = torch.from_numpy(A).to(dev)
    dB = torch.from_numpy(B).to(dev)
    ldc = N + ldc_pad
    dC = torch.full((M * ldc + 1,), float("nan"), device=dev)
    ws = torch.full((max(1, ws_bytes // 4),), float("nan"), device=dev)
    say(f"gemm_f32_ws M={M} N={N} K={K} workspace {ws_bytes} of {need} bytes")
    rc = gb.gemm_f32_ws(M, N, K, dA.data_ptr(), K, dB.data_ptr(), N, dC.data_ptr(), ldc,
                        ws.data_ptr(), ws_bytes, torch.cuda.current_stream().cuda_stream)
    assert rc == gb.GEMM_F32_OK, gb.gemm_f32_status_string(rc)
    torch.cuda.synchronize()
    full = dC.cpu().numpy()
    return np.ascontiguousarray(full[:M * ldc].reshape(M, ldc)[:, :N]), full, ws.cpu().numpy(), need


SPLITK = [(200, 200, 20000), (130, 70, 5000), (64, 300, 3000), (17, 1000, 4096), (600, 600, 4096),
          (640, 650, 8190)]


@pytest.mark.parametrize("shape", SPLITK, ids=lambda s: "x".join(map(str, s)))
def test_split_k_bit_exact_and_padding_kept(dev, shape):
    A, B = operands("quarter", *shape)
    got, full, _, need = gpu_gemm_ws(A, B, dev, ldc_pad=3)
    assert need > 0
    assert_bit_exact(got, oracle.gemm(A, B), f"{shape} split-K")
    M, N, _ = shape
    body = full[:M * (N + 3)].reshape(M, N + 3)
    assert np.isnan(body[:, N:]).all() and np.isnan(full[-1])


def test_split_k_uniform_within_tolerance_and_deterministic(dev):
    A, B = operands("uniform", 200, 200, 20000)
    first, _, _, _ = gpu_gemm_ws(A, B, dev)
    assert_close(first, oracle.gemm(A, B), "200x200x20000 split-K")
    for _ in range(2):
        again, _, _, _ = gpu_gemm_ws(A, B, dev)
        assert_bit_exact(again, first, "split-K repeat")


def test_split_k_special_values_classified_as_the_oracle(dev):
    """The slices' partial products and their ordered sum keep NaN and
    +-Inf where the oracle has them."""
    A, B = special_operands(200, 200, 20000, count=12)
    got, _, _, need = gpu_gemm_ws(A, B, dev)
    assert need > 0
    with np.errstate(invalid="ignore"):
        ref = oracle.gemm(A, B)
    for f in (np.isnan, np.isposinf, np.isneginf):
        assert np.array_equal(f(got), f(ref)), f.__name__
    fin = np.isfinite(ref)
    assert fin.any() and not fin.all()
    assert_close(got[fin], ref[fin], "split-K special finite part")


def test_split_k_short_workspace_runs_the_plain_path(dev):
    """Too small a workspace: the call is gemm_f32's and the workspace is
    not touched."""
    A, B = operands("quarter", 130, 70, 5000)
    got, _, ws, need = gpu_gemm_ws(A, B, dev, ws_bytes=1 << 12)
    assert need > (1 << 12)
    assert_bit_exact(got, oracle.gemm(A, B), "short workspace")
    assert np.isnan(ws).all()


@pytest.mark.parametrize("config", [c for c in CONFIGS if gb.gemm_f32_config_name(c).startswith("dma")],
                         ids=[n for n in CONFIG_IDS if n.startswith("dma")])
def test_a_chunks_crossing_column_k_are_cleared(dev, config):
    """K % 4 != 0 with NaN in A's row padding (and after A's last element):
    the 128-bit A chunk holding column K-1 picks those up in LDS, where they
    must be cleared before they meet B's zero rows (NaN * 0 would be NaN)."""
    for M, N, K in ((130, 200, 77), (300, 128, 131), (64, 64, 5)):
        A, B = operands("quarter", M, N, K)
        for pad, off in (((0, 0, 0), (0, 0, 0)), ((3, 0, 0), (0, 0, 0)), ((1, 2, 0), (3, 1, 0))):
            got, _ = gpu_gemm(A, B, config, dev, pad=pad, offset=off)
            assert_bit_exact(got, oracle.gemm(A, B), f"{(M, N, K)} pad {pad} off {off}")


def test_split_k_in_graph(dev):
    """The split-K plan is two kernels (slices into the workspace, then the
    ordered sum) and no memset: captured into a HIP graph, every replay
    reproduces the eager result bit for bit."""
    M, N, K = 200, 200, 20000
    A, B = operands("uniform", M, N, K)
    dA = torch.from_numpy(A).to(dev)
    dB = torch.from_numpy(B).to(dev)
    need = gb.gemm_f32_ws_size(M, N, K)
    ws = torch.empty(need // 4, device=dev)
    out = torch.full((M, N), float("nan"), device=dev)

    def call(stream):
        return gb.gemm_f32_ws(M, N, K, dA.data_ptr(), K, dB.data_ptr(), N, out.data_ptr(), N,
                              ws.data_ptr(), need, stream.cuda_stream)

    say("split-K eager and graph, 200x200x20000")
    assert call(torch.cuda.current_stream()) == gb.GEMM_F32_OK
    torch.cuda.synchronize()
    eager = out.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        call(s)
    for _ in range(3):
        out.fill_(float("nan"))
        ws.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager)
