"""The C ABI of libgemm_f32.so: exports, argument validation, plan description.

The CPU tests here never launch a kernel: every call either fails validation
or has an empty output, which the library handles on the host before any HIP
call.  Launching tests are marked ``gpu``.
"""
import re
import os

import numpy as np
import pytest

from dense_fp32_gemm_amd import binding as gb

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gemm_f32.h")

FAKE = 0x100000   # a 4-byte aligned address that is never dereferenced


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"GEMM_F32_API\s+[\w\s\*]*?\b(gemm_f32\w*)\s*\(", text)))


def test_library_exports_every_declared_function():
    names = declared_functions()
    assert "gemm_f32" in names and len(names) >= 6
    lib = gb.load()
    for n in names:
        assert hasattr(lib, n), n
        assert hasattr(gb, n), f"binding lacks {n}"


def test_status_codes_match_header():
    text = open(HEADER).read()
    for name, value in re.findall(r"#define (GEMM_F32_(?:OK|ERR_\w+))\s+(\d+)", text):
        assert getattr(gb, name) == int(value), name
        assert gb.gemm_f32_status_string(int(value)) not in ("", "unknown status")


def test_config_names():
    names = gb.config_names()
    assert len(names) == gb.gemm_f32_num_configs() >= 2
    assert names[0].startswith("valu") and any(n.startswith("dma") for n in names)
    assert any(n.startswith("staged") for n in names)
    assert gb.gemm_f32_config_name(-1) == "" and gb.gemm_f32_config_name(len(names)) == ""


@pytest.mark.parametrize("M,N,K", [(-1, 4, 4), (4, -1, 4), (4, 4, -1)])
def test_negative_sizes(M, N, K):
    assert gb.gemm_f32(M, N, K, FAKE, 4, FAKE, 4, FAKE, 4, 0) == gb.GEMM_F32_ERR_DIM


@pytest.mark.parametrize("lda,ldb,ldc", [(7, 9, 9), (8, 8, 9), (8, 9, 8), (0, 9, 9)])
def test_small_leading_dimension(lda, ldb, ldc):
    assert gb.gemm_f32(5, 9, 8, FAKE, lda, FAKE, ldb, FAKE, ldc, 0) == gb.GEMM_F32_ERR_LD


def test_leading_dimension_minimum_is_one():
    # K == 0 still needs lda >= 1; N == 0 still needs ldb, ldc >= 1.
    assert gb.gemm_f32(3, 0, 0, 0, 0, 0, 1, 0, 1, 0) == gb.GEMM_F32_ERR_LD
    assert gb.gemm_f32(3, 0, 2, 0, 2, 0, 0, 0, 1, 0) == gb.GEMM_F32_ERR_LD


def test_null_pointers():
    assert gb.gemm_f32(4, 4, 4, 0, 4, FAKE, 4, FAKE, 4, 0) == gb.GEMM_F32_ERR_NULL
    assert gb.gemm_f32(4, 4, 4, FAKE, 4, 0, 4, FAKE, 4, 0) == gb.GEMM_F32_ERR_NULL
    assert gb.gemm_f32(4, 4, 4, FAKE, 4, FAKE, 4, 0, 4, 0) == gb.GEMM_F32_ERR_NULL
    assert gb.gemm_f32(4, 4, 0, 0, 1, 0, 4, 0, 4, 0) == gb.GEMM_F32_ERR_NULL   # K=0 still writes C


def test_misaligned_pointers():
    assert gb.gemm_f32(4, 4, 4, FAKE + 2, 4, FAKE, 4, FAKE, 4, 0) == gb.GEMM_F32_ERR_ALIGN
    assert gb.gemm_f32(4, 4, 4, FAKE, 4, FAKE + 1, 4, FAKE, 4, 0) == gb.GEMM_F32_ERR_ALIGN
    assert gb.gemm_f32(4, 4, 4, FAKE, 4, FAKE, 4, FAKE + 3, 4, 0) == gb.GEMM_F32_ERR_ALIGN


def test_validation_order():
    # sizes, leading dimensions, configuration, pointers, alignment -- the
    # order include/gemm_f32.h states
    bad = gb.gemm_f32_num_configs()
    assert gb.gemm_f32(-1, 4, 4, 0, 0, 0, 0, 0, 0, 0) == gb.GEMM_F32_ERR_DIM
    assert gb.gemm_f32_with_config(bad, -1, 4, 4, 0, 0, 0, 0, 0, 0, 0) == gb.GEMM_F32_ERR_DIM
    assert gb.gemm_f32(4, 4, 4, 0, 0, 0, 4, 0, 4, 0) == gb.GEMM_F32_ERR_LD
    assert gb.gemm_f32_with_config(bad, 4, 4, 4, 0, 0, 0, 4, 0, 4, 0) == gb.GEMM_F32_ERR_LD
    assert gb.gemm_f32_with_config(bad, 4, 4, 4, 0, 4, 0, 4, 0, 4, 0) == gb.GEMM_F32_ERR_CONFIG
    assert gb.gemm_f32_with_config(bad, 0, 4, 4, 0, 4, 0, 4, 0, 4, 0) == gb.GEMM_F32_ERR_CONFIG
    assert gb.gemm_f32(4, 4, 4, 0, 4, FAKE + 1, 4, FAKE, 4, 0) == gb.GEMM_F32_ERR_NULL
    assert gb.gemm_f32(4, 4, 4, FAKE + 1, 4, FAKE, 4, FAKE, 4, 0) == gb.GEMM_F32_ERR_ALIGN


def test_unknown_config():
    n = gb.gemm_f32_num_configs()
    for c in (-2, n, n + 7):
        assert gb.gemm_f32_with_config(c, 4, 4, 4, FAKE, 4, FAKE, 4, FAKE, 4, 0) == gb.GEMM_F32_ERR_CONFIG


@pytest.mark.parametrize("M,N", [(0, 5), (5, 0), (0, 0)])
def test_empty_output_is_ok_without_pointers(M, N):
    assert gb.gemm_f32(M, N, 7, 0, 7, 0, max(N, 1), 0, max(N, 1), 0) == gb.GEMM_F32_OK


def test_describe():
    rc, text = gb.gemm_f32_describe(-1, 0, 5, 3, 0, 3, 0, 5, 0, 5)
    assert rc == gb.GEMM_F32_OK and text == "none"
    rc, text = gb.gemm_f32_describe(-1, 5, 5, 0, 0, 1, 0, 5, FAKE, 5)
    assert rc == gb.GEMM_F32_OK and text == "fill_zero"
    rc, text = gb.gemm_f32_describe(-1, -1, 5, 3, 0, 3, 0, 5, 0, 5)
    assert rc == gb.GEMM_F32_ERR_DIM and text.startswith("invalid")
    rc, text = gb.gemm_f32_describe(-1, 8192, 8192, 8192, FAKE, 8192, FAKE, 8192, FAKE, 8192)
    assert rc == gb.GEMM_F32_OK and text.startswith("dma") and "load_a=x4 load_b=x4" in text
    # direct-to-LDS loads: 128-bit from any 4-byte aligned address, for any K
    rc, text = gb.gemm_f32_describe(-1, 1025, 1023, 1000, FAKE, 1000, FAKE, 1023, FAKE, 1023)
    assert rc == gb.GEMM_F32_OK and "load_a=x4 load_b=x4" in text
    rc, text = gb.gemm_f32_describe(-1, 512, 512, 512, FAKE + 4, 515, FAKE + 8, 517, FAKE, 512)
    assert text.startswith("dma") and "load_a=x4 load_b=x4" in text, text
    rc, text = gb.gemm_f32_describe(-1, 512, 512, 1001, FAKE, 1001, FAKE, 512, FAKE, 512)
    assert text.startswith("dma") and "load_a=x4 load_b=x4" in text, text
    rc, text = gb.gemm_f32_describe(-1, 1, 1, 1, FAKE, 1, FAKE, 1, FAKE, 1)
    assert rc == gb.GEMM_F32_OK and text.startswith("valu")
    # the register-staged kernel keeps 16-byte alignment for its 128-bit loads
    staged = gb.config_names().index("staged_64x64x16")
    rc, text = gb.gemm_f32_describe(staged, 512, 512, 512, FAKE + 4, 512, FAKE, 512, FAKE, 512)
    assert "load_a=x1 load_b=x4" in text, text


WRITE_BACK = ["dma_64x64x32", "dma_64x128x32", "dma_128x64x32", "dma_64x64x32_sk",
              "dma_256x256x32_pipe", "dma_256x256x32_pipe_sk", "dma_128x128x64_pipe_lw2",
              "dma_128x128x64_pipe_lw2_sk", "dma_64x64x16_ksplit8_pipe",
              "dma_128x128x16_pipe", "dma_128x128x32_pipe"]


def test_describe_write_back_c_stores():
    """C with at least 2^23 elements and rows that are not 16-byte aligned
    (ldc % 4 != 0, or a base 4 bytes off) runs the write-back twin of the
    chosen tile; aligned rows, a smaller C or a tile without a twin stream."""
    rc, text = gb.gemm_f32_describe(-1, 4119, 4789, 77, FAKE, 77, FAKE, 4789, FAKE, 4789)
    assert rc == gb.GEMM_F32_OK and text.endswith("c_store=write_back"), text
    rc, text = gb.gemm_f32_describe(-1, 4096, 4096, 77, FAKE, 77, FAKE, 4096, FAKE + 8, 4096)
    assert text.endswith("c_store=write_back"), text
    rc, text = gb.gemm_f32_describe(-1, 4096, 4096, 77, FAKE, 77, FAKE, 4096, FAKE, 4096)
    assert "write_back" not in text, text
    rc, text = gb.gemm_f32_describe(-1, 2048, 4095, 77, FAKE, 77, FAKE, 4095, FAKE, 4095)
    assert "write_back" not in text, text          # 2048 * 4095 < 2^23 elements
    rc, text = gb.gemm_f32_describe(-1, 2049, 4097, 40, FAKE, 40, FAKE, 4097, FAKE, 4097)
    assert text.endswith("c_store=write_back"), text
    names = gb.config_names()
    for c, n in enumerate(names):
        rc, text = gb.gemm_f32_describe(c, 2049, 4097, 40, FAKE, 40, FAKE, 4097, FAKE, 4097)
        assert rc == gb.GEMM_F32_OK
        assert ("c_store=write_back" in text) == (n in WRITE_BACK), (n, text)


def test_wide_rows_fall_back_to_staged_kernels():
    """Direct-to-LDS kernels address a panel with 32-bit offsets; rows so long
    that a panel spans 2 GiB select the register-staged kernels instead, and
    forcing a direct-to-LDS configuration is refused."""
    lda = 1 << 26                      # 128 rows of A span 32 GiB
    rc, text = gb.gemm_f32_describe(-1, 4096, 4096, 1000, FAKE, lda, FAKE, 4096, FAKE, 4096)
    assert rc == gb.GEMM_F32_OK and text.startswith("staged"), text
    dma = [i for i, n in enumerate(gb.config_names()) if n.startswith("dma")]
    for c in dma:
        rc, _ = gb.gemm_f32_describe(c, 4096, 4096, 1000, FAKE, lda, FAKE, 4096, FAKE, 4096)
        assert rc == gb.GEMM_F32_ERR_CONFIG
    ldb = 1 << 27                      # 16 rows of B span 8 GiB
    rc, text = gb.gemm_f32_describe(-1, 4096, 4096, 1000, FAKE, 1000, FAKE, ldb, FAKE, 4096)
    assert text.startswith("staged"), text
    # 63 rows of B span more than 2 GiB but 31 do not: the rule's 64-deep
    # choices give way to its 32-deep ones
    ldb = 10_000_000
    rc, text = gb.gemm_f32_describe(-1, 1400, 1400, 1000, FAKE, 1000, FAKE, ldb, FAKE, 1400)
    assert rc == gb.GEMM_F32_OK and text.startswith("dma_64x64x32 "), text
    rc, text = gb.gemm_f32_describe(-1, 2048, 2048, 2048, FAKE, 2048, FAKE, ldb, FAKE, 2048)
    assert rc == gb.GEMM_F32_OK and text.startswith("dma_128x128x32_ksplit2 "), text
    rc, text = gb.gemm_f32_describe(-1, 3072, 3072, 3072, FAKE, 3072, FAKE, ldb, FAKE, 3072)
    assert rc == gb.GEMM_F32_OK and text.startswith("dma_128x128x32_w16_sk "), text
    rc, text = gb.gemm_f32_describe(-1, 1100, 1100, 1300, FAKE, 1300, FAKE, ldb, FAKE, 1100)
    assert rc == gb.GEMM_F32_OK and text.startswith("dma_64x64x16_ksplit8_pipe_sk "), text
    rc, text = gb.gemm_f32_describe(-1, 1025, 1023, 1000, FAKE, 1000, FAKE, ldb, FAKE, 1023)
    assert rc == gb.GEMM_F32_OK and text.startswith("dma_64x64x16_ksplit8_pipe ") and "strip_rows=1" in text, text
    rc, text = gb.gemm_f32_describe(-1, 1023, 1025, 256, FAKE, 256, FAKE, ldb, FAKE, 1025)
    assert rc == gb.GEMM_F32_OK and text.startswith("dma_64x64x32 "), text
    k64 = gb.config_names().index("dma_64x64x64")
    rc, _ = gb.gemm_f32_describe(k64, 1024, 1024, 1024, FAKE, 1024, FAKE, ldb, FAKE, 1024)
    assert rc == gb.GEMM_F32_ERR_CONFIG


@pytest.mark.parametrize("shape,name", [
    ((8192, 8192, 8192), "dma_256x256x32_pipe "), ((2048, 2048, 2048), "dma_128x128x64_pipe_lw2 "),
    ((4096, 4096, 16384), "dma_256x256x32_pipe "), ((1024, 8192, 8192), "dma_128x128x32_pipe "),
    ((8192, 8192, 128), "dma_128x128x16_pipe "), ((8192, 8192, 512), "dma_128x128x16_pipe "),
    ((1, 1, 1), "valu"), ((15, 4000, 4000), "valu"),
    # at most one 64 x 64 tile per CU: 8 pipelined one-wave K-split groups
    # from K = 640 on, unless below K = 1536 the 16-deep panels split
    # unevenly over the groups (the busiest group's share of K rounded up
    # over 9/8 of K rounded up to 32); otherwise 4 waves fed by two loader
    # waves
    ((16384, 64, 4096), "dma_64x64x16_ksplit8_pipe "), ((64, 16384, 4096), "dma_64x64x16_ksplit8_pipe "),
    ((1024, 1024, 8192), "dma_64x64x16_ksplit8_pipe "), ((100, 5000, 3000), "dma_64x64x16_ksplit8_pipe "),
    ((1024, 1024, 1536), "dma_64x64x16_ksplit8_pipe "), ((1000, 1000, 1535), "dma_64x64x16_ksplit8_pipe "),
    ((1000, 1000, 1000), "dma_64x64x16_ksplit8_pipe "), ((768, 768, 1024), "dma_64x64x16_ksplit8_pipe "),
    ((1024, 1024, 640), "dma_64x64x16_ksplit8_pipe "), ((1000, 1000, 700), "dma_64x64x16_ksplit8_pipe "),
    ((1024, 1024, 512), "dma_64x64x16_ksplit8_pipe "), ((1000, 1000, 400), "dma_64x64x16_ksplit8_pipe "),
    ((960, 1000, 350), "dma_64x64x32 "),
    ((800, 1200, 650), "dma_64x64x32_pipe_lw2_s4 "), ((1000, 1000, 639), "dma_64x64x32_pipe_lw2_s4 "),
    ((1000, 1000, 600), "dma_64x64x32_pipe_lw2_s4 "), ((1000, 1000, 513), "dma_64x64x32_pipe_lw2_s4 "),
    # K <= 512: no K split; 64-deep panels unless the last one would be at
    # most half used (K % 64 in 1..32)
    ((1000, 1000, 300), "dma_64x64x64 "), ((1280, 1280, 512), "dma_64x64x64 "),
    ((600, 3000, 200), "dma_64x64x32 "), ((956, 1597, 331), "dma_64x64x32 "),
    ((2712, 228, 94), "dma_64x64x32 "),
    # few output tiles: 32 x 32 tiles of one-wave K-split groups while they
    # fit one round (4 groups for K <= 256), then 32 x 64 or 64 x 32 ones
    ((512, 512, 512), "dma_32x32x32_ksplit8 "), ((512, 512, 1024), "dma_32x32x32_ksplit8 "),
    ((256, 256, 8192), "dma_32x32x32_ksplit8 "), ((17, 33, 65), "dma_32x32x32_ksplit4 "),
    ((300, 400, 100), "dma_32x32x32_ksplit4 "), ((64, 2048, 2048), "dma_32x32x32_ksplit8 "),
    ((640, 640, 2048), "dma_32x64x16_ksplit8 "), ((512, 1024, 1024), "dma_32x64x16_ksplit8 "),
    ((1024, 512, 1024), "dma_32x64x16_ksplit8 "), ((700, 600, 1000), "dma_32x64x16_ksplit8 "),
    ((960, 544, 1000), "dma_64x32x16_ksplit8 "),
    # 272 tiles, 16 of them for a last row of 1-4 rows (rows x K <= 4096): one
    # round of K-split tiles and a strip of FMAs
    ((1025, 1023, 1000), "dma_64x64x16_ksplit8_pipe "), ((1028, 1000, 1000), "dma_64x64x16_ksplit8_pipe "),
    ((1025, 1023, 2048), "dma_64x64x16_ksplit8_pipe "), ((1025, 1023, 3000), "dma_64x64x16_ksplit8_pipe "),
    ((1023, 1025, 1000), "dma_64x64x16_ksplit8_pipe "), ((1025, 1025, 1000), "dma_64x64x16_ksplit8_pipe "),
    ((1025, 1025, 3072), "dma_64x64x16_ksplit8_pipe "),
    # just past one round with K < 1536 (rows x K over 4096): stream-K over
    # the 4-group K split
    ((1028, 1000, 1500), "dma_64x64x32_ksplit4_sk "), ((1029, 1025, 1200), "dma_64x64x32_ksplit4_sk "),
    # 289, 324, 441 and 576 64 x 64 tiles: the idle CU-rounds times K are
    # large enough for stream-K over the 8 pipelined groups.  400 tiles (a
    # last round 56 % full) with K = 1280: two rounds of the 8 groups
    ((1025, 1025, 4096), "dma_64x64x16_ksplit8_pipe_sk "),
    ((1100, 1100, 1100), "dma_64x64x16_ksplit8_pipe_sk "), ((1300, 1300, 4096), "dma_64x64x16_ksplit8_pipe_sk "),
    ((1536, 1536, 1536), "dma_64x64x16_ksplit8_pipe_sk "), ((1280, 1280, 1280), "dma_64x64x16_ksplit8_pipe "),
    ((1025, 1023, 300), "dma_64x64x16_ksplit8_pipe "), ((1023, 1025, 256), "dma_64x64x64 "),
    ((1590, 744, 100), "dma_64x64x32 "),
    # two balanced rounds: the pipelined K split for K >= 1024, else 64 x 64
    ((2048, 1024, 1024), "dma_64x64x16_ksplit8_pipe "),
    ((1400, 1400, 1000), "dma_64x64x64 "), ((2048, 1024, 768), "dma_64x64x64 "),
    # three rounds: the pipelined K split for K >= 2048; more rounds: 4-wave
    # 64 x 64 tiles, several per CU
    ((3072, 1024, 2048), "dma_64x64x16_ksplit8_pipe "), ((1900, 1600, 1500), "dma_64x64x32 "),
    ((2176, 2100, 1000), "dma_64x64x32 "),
    # 400, 576, 1600 and 1849 128 x 128 tiles, K >= 2048: stream-K over them
    # (under two rounds of 256 x 256 tiles); 728 256 x 256 tiles with K >=
    # 3072, 2912 128 x 128 ones: stream-K over the 256 x 256 tiles
    ((2560, 2560, 2560), "dma_128x128x64_pipe_lw2_sk "), ((3072, 3072, 3072), "dma_128x128x64_pipe_lw2_sk "),
    ((5000, 5000, 5000), "dma_128x128x64_pipe_lw2_sk "), ((5500, 5500, 3500), "dma_128x128x64_pipe_lw2_sk "),
    ((7168, 6656, 4096), "dma_256x256x32_pipe_sk "),
    # two or more balanced rounds of 128 x 128 tiles: 16-deep pipelined
    # panels for K < 2048
    ((6000, 2000, 1000), "dma_128x128x16_pipe "), ((4096, 3072, 1024), "dma_128x128x16_pipe "),
    ((4096, 2048, 2048), "dma_128x128x32_pipe "), ((4096, 2048, 1024), "dma_128x128x32_pipe "),
    ((6144, 2048, 4096), "dma_128x128x16_pipe "), ((2048, 2048, 1024), "dma_128x128x64_pipe_lw2 "),
    # a side of at most 64 (or 129 to 192): 128-wide tiles would be mostly
    # padding, so only the 64 x 64 choices; a side of 96 or 128 keeps them
    ((64, 32768, 4096), "dma_64x64x16_ksplit8_pipe "), ((32768, 64, 4096), "dma_64x64x16_ksplit8_pipe "),
    ((192, 16384, 4096), "dma_64x64x16_ksplit8_pipe "), ((64, 32768, 1024), "dma_64x64x16_ksplit8_pipe "),
    ((64, 65536, 1024), "dma_64x64x32 "), ((65536, 64, 1024), "dma_64x64x32 "),
    ((96, 32768, 4096), "dma_128x128x64_pipe_lw2 "), ((128, 32768, 4096), "dma_128x128x64_pipe_lw2 "),
    # a second round exactly half full (384 tiles): stream-K over the 8
    # pipelined groups
    ((64, 24576, 4096), "dma_64x64x16_ksplit8_pipe_sk "), ((128, 12288, 12000), "dma_64x64x16_ksplit8_pipe_sk "),
    # unless 64-wide tiles pad a side under 192 by a third more than 32-wide
    # ones: 32 x 64 (64 x 32) tiles of the 8-group K split
    ((95, 8926, 1248), "dma_32x64x16_ksplit8 "), ((8926, 95, 1248), "dma_64x32x16_ksplit8 "),
    ((80, 12000, 2000), "dma_32x64x16_ksplit8 "), ((96, 8192, 1024), "dma_64x64x16_ksplit8_pipe "),
    ((15133, 90, 3196), "dma_64x32x16_ksplit8 "),
    # 196 128 x 128 tiles against 784 64 x 64 ones (a fourth round barely used)
    ((1792, 1792, 1792), "dma_128x128x64_pipe_lw2 "),
    # past one round of 64 x 64 tiles, 32 x 64 (64 x 32) ones that fill at
    # most two rounds, for 256 < K < 2560; stream-K over the 8 pipelined
    # groups from there, two rounds of 64 x 64 tiles below
    ((535, 1913, 2314), "dma_32x64x16_ksplit8 "), ((4157, 207, 1519), "dma_64x32x16_ksplit8 "),
    ((535, 1913, 450), "dma_32x64x16_ksplit8 "), ((535, 1913, 256), "dma_64x64x64 "),
    ((1000, 1000, 300), "dma_64x64x64 "),
    ((1620, 634, 695), "dma_32x64x16_ksplit8 "), ((1247, 792, 4980), "dma_64x64x16_ksplit8_pipe_sk "),
    # four to six rounds of 64 x 64 tiles where the 128 x 128 choices do not
    # apply: stream-K over the 8 pipelined groups where it pays
    ((198, 16642, 1898), "dma_64x64x16_ksplit8_pipe_sk "), ((29205, 160, 3003), "dma_64x64x16_ksplit8_pipe_sk "),
    ((42104, 99, 1696), "dma_64x64x16_ksplit8_pipe_sk "), ((1500, 3500, 1050), "dma_64x64x32 "),
    # just past one round of 64 x 64 tiles with K < 1150: 32 x 32 tiles of 4
    # K-split groups
    ((309, 3485, 597), "dma_32x32x32_ksplit4 "), ((660, 1684, 979), "dma_32x32x32_ksplit4 "),
    ((574, 1850, 1256), "dma_64x64x32_ksplit4_sk "),
    # 198-249 128 x 128 tiles where 64 x 64 tiles take four rounds: one
    # round of 128 x 128, 32-deep panels if a 64-deep last one would be at
    # most half used; three rounds of 64 x 64 tiles: those
    ((3394, 1064, 960), "dma_128x128x64_pipe_lw2 "), ((2282, 1391, 771), "dma_128x128x32_pipe "),
    ((1800, 1800, 2500), "dma_128x128x64_pipe_lw2 "), ((2000, 1700, 4000), "dma_128x128x64_pipe_lw2 "),
    # unless the fourth round of 64 x 64 tiles is nearly empty and K long:
    # stream-K over the 8 pipelined groups
    ((1664, 1950, 11185), "dma_64x64x16_ksplit8_pipe_sk "), ((1700, 1900, 5000), "dma_64x64x16_ksplit8_pipe_sk "),
    ((1551, 1838, 1619), "dma_64x64x32 "), ((3072, 1024, 2048), "dma_64x64x16_ksplit8_pipe "),
    # 486 128 x 128 tiles (a second round 90 % full) with 1024 <= K < 2048:
    # two rounds of the 32-deep pipelined tile; 324 (27 % full): 64 x 64
    ((3428, 2297, 1956), "dma_128x128x32_pipe "), ((2200, 2200, 1500), "dma_64x64x32 "),
])
def test_selection(shape, name):
    M, N, K = shape
    rc, text = gb.gemm_f32_describe(-1, M, N, K, FAKE, K, FAKE, N, FAKE, N)
    assert rc == gb.GEMM_F32_OK and text.startswith(name), text


def test_config_info_matches_names():
    for c, name in enumerate(gb.config_names()):
        info = gb.gemm_f32_config_info(c)
        tile = name.split("_")[1]                      # e.g. "256x256x16" or "64x64"
        dims = [int(x) for x in tile.split("x")]
        assert [info["bm"], info["bn"]] == dims[:2], name
        if len(dims) == 3:
            assert info["bk"] == dims[2], name
        assert info["threads"] % 64 == 0 and 64 <= info["threads"] <= 1024
    with pytest.raises(gb.GemmError):
        gb.gemm_f32_config_info(gb.gemm_f32_num_configs())


def test_device_peak_without_a_device_is_an_error():
    torch = pytest.importorskip("torch")
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    with pytest.raises(gb.GemmError):
        gb.gemm_f32_device_peak(0)


def test_streamk_grid_is_one_worker_per_compute_unit():
    cfg = gb.config_names().index("dma_64x64x64_sk")
    rc, text = gb.gemm_f32_describe(cfg, 1025, 1023, 1000, FAKE, 1000, FAKE, 1023, FAKE, 1023)
    assert rc == gb.GEMM_F32_OK and "tiles=17x16 grid=256 " in text, text
    # fewer tiles than compute units: one worker per tile, nothing shared
    rc, text = gb.gemm_f32_describe(cfg, 300, 300, 1000, FAKE, 1000, FAKE, 300, FAKE, 300)
    assert rc == gb.GEMM_F32_OK and "tiles=5x5 grid=25 " in text, text


def test_split_k_workspace_size():
    # 200 x 200: 16 tiles of 64 x 64 -> 16 slices of a 20000-deep K
    assert gb.gemm_f32_ws_size(200, 200, 20000) == 16 * 200 * 200 * 4
    # slices also limited by K: 32 panels of 32 -> at most 4 slices of 8 panels
    assert gb.gemm_f32_ws_size(64, 64, 1024) == 4 * 64 * 64 * 4
    # 100 tiles fill up to 2 slices
    assert gb.gemm_f32_ws_size(640, 640, 8192) == 2 * 640 * 640 * 4
    # enough tiles, too short a K, tiny or invalid shapes: not split
    for shape in [(8192, 8192, 8192), (2048, 2048, 2048), (1024, 1024, 8192), (64, 64, 256),
                  (200, 200, 0), (8, 8, 100000), (-1, 200, 20000)]:
        assert gb.gemm_f32_ws_size(*shape) == 0, shape


def test_split_k_entry_point_validates_like_gemm_f32():
    ws = 1 << 20
    assert gb.gemm_f32_ws(-1, 4, 4, FAKE, 4, FAKE, 4, FAKE, 4, FAKE, ws, 0) == gb.GEMM_F32_ERR_DIM
    assert gb.gemm_f32_ws(5, 9, 8, FAKE, 7, FAKE, 9, FAKE, 9, FAKE, ws, 0) == gb.GEMM_F32_ERR_LD
    assert gb.gemm_f32_ws(5, 9, 8, 0, 8, FAKE, 9, FAKE, 9, FAKE, ws, 0) == gb.GEMM_F32_ERR_NULL
    assert gb.gemm_f32_ws(0, 9, 8, 0, 8, 0, 9, 0, 9, 0, 0, 0) == gb.GEMM_F32_OK


def test_traffic_records_key_on_code_not_comments(tmp_path):
    import bench
    a = tmp_path / "a.hip"
    a.write_text("int f(int x)\n{\n    return x + 1;   // one more\n}\n")
    b = tmp_path / "b.hip"
    b.write_text("// a new comment line\nint f(int x)\n{\n\n    return x + 1;   // one more, said again\n}\n")
    c = tmp_path / "c.hip"
    c.write_text("int f(int x)\n{\n    return x + 2;\n}\n")
    assert bench.code_digest(a) == bench.code_digest(b) != bench.code_digest(c)


def test_strip_width_never_exceeds_four():
    """The strip kernel sums 1-4 rows (columns).  Sweep shapes around one
    round of 64 x 64 tiles, where strips are planned, over K from just past
    512 to the strip limit: every planned strip is at most 4 wide, and a
    remainder of 5-63 rows or columns is never a strip."""
    seen, both = set(), set()
    for base_m, base_n in ((1024, 1000), (1000, 1024), (960, 1088), (1088, 960), (1024, 1024)):
        for rem in range(0, 64):
            for K in (256, 257, 400, 513, 600, 700, 819, 820, 1000, 1023, 1024, 1365, 2047, 3072, 4096):
                for M, N in ((base_m + rem, base_n), (base_m, base_n + rem), (base_m + rem, base_n + rem % 5)):
                    rc, text = gb.gemm_f32_describe(-1, M, N, K, FAKE, K, FAKE, N, FAKE, N)
                    assert rc == gb.GEMM_F32_OK, (M, N, K, text)
                    found = re.findall(r"strip_(rows|cols)=(\d+)", text)
                    for side, width in found:
                        width = int(width)
                        assert 1 <= width <= 4, (M, N, K, text)
                        assert width == (M % 64 if side == "rows" else N % 64), (M, N, K, text)
                        assert width * K <= 4096, (M, N, K, text)
                        seen.add((side, width))
                    if len(found) == 2:
                        assert K <= 3072, (M, N, K, text)
                        both.add((M % 64, N % 64))
    # the sweep does reach strips of every width on both sides, and pairs
    assert seen == {(side, w) for side in ("rows", "cols") for w in (1, 2, 3, 4)}, seen
    assert {(1, 1), (2, 2), (3, 3), (4, 4)} <= both, both


def test_sizes_beyond_a_c_int_are_refused_before_the_call():
    """ctypes would wrap 2^32 + 1000 to 1000; the binding raises instead."""
    big = (1 << 32) + 1000
    with pytest.raises(ValueError):
        gb.gemm_f32(big, 4, 4, FAKE, 4, FAKE, 4, FAKE, 4, 0)
    with pytest.raises(ValueError):
        gb.gemm_f32(4, 4, 4, FAKE, big, FAKE, 4, FAKE, 4, 0)
    with pytest.raises(ValueError):
        gb.gemm_f32_with_config(-1, 4, 4, 4, FAKE, 4, FAKE, 4, FAKE, 1 << 31, 0)
    with pytest.raises(ValueError):
        gb.gemm_f32_ws(4, 4, big, FAKE, 4, FAKE, 4, FAKE, 4, FAKE, 1 << 20, 0)
    with pytest.raises(ValueError):
        gb.gemm_f32_ws_size(4, -(1 << 31) - 1, 4)
    with pytest.raises(ValueError):
        gb.gemm_f32_describe(-1, 4, 4, 4, FAKE, 4, FAKE, big, FAKE, 4)
    # the extremes a C int holds still reach the library
    assert gb.gemm_f32(-(1 << 31), 4, 4, FAKE, 4, FAKE, 4, FAKE, 4, 0) == gb.GEMM_F32_ERR_DIM
    assert gb.gemm_f32(4, 4, 4, FAKE, (1 << 31) - 1, FAKE, 4, FAKE, 3, 0) == gb.GEMM_F32_ERR_LD


def test_describe_names_plans_that_add_into_c():
    """Stream-K plans whose workers split a tile's K-panels sum that tile in C
    with atomic adds (C must be ordinary device memory); describe says so."""
    rc, text = gb.gemm_f32_describe(-1, 1029, 1025, 1200, FAKE, 1200, FAKE, 1025, FAKE, 1025)
    assert rc == gb.GEMM_F32_OK and "_sk " in text and text.endswith(" c_accumulate=atomic_add"), text
    sk = gb.config_names().index("dma_64x64x64_sk")
    # fewer tiles than workers: one worker per tile, nothing shared
    rc, text = gb.gemm_f32_describe(sk, 300, 300, 1000, FAKE, 1000, FAKE, 300, FAKE, 300)
    assert "grid=25 " in text and "atomic" not in text, text
    # 512 tiles, 64 panels each, over 256 workers: every range is two whole tiles
    rc, text = gb.gemm_f32_describe(sk, 1024, 2048, 4096, FAKE, 4096, FAKE, 2048, FAKE, 2048)
    assert "tiles=16x32 grid=256 " in text and "atomic" not in text, text
    for shape in [(8192, 8192, 8192), (2048, 2048, 2048), (1000, 1000, 1000), (1025, 1023, 1000)]:
        M, N, K = shape
        rc, text = gb.gemm_f32_describe(-1, M, N, K, FAKE, K, FAKE, N, FAKE, N)
        assert "atomic" not in text, text
    # with the write-back twin both markers appear
    wb_sk = gb.config_names().index("dma_64x64x32_sk")
    rc, text = gb.gemm_f32_describe(wb_sk, 2049, 4097, 40, FAKE, 40, FAKE, 4097, FAKE, 4097)
    assert text.endswith(" c_store=write_back c_accumulate=atomic_add"), text


def test_noalloc_entry_point_validates_like_gemm_f32():
    f = gb.gemm_f32_ws_noalloc
    assert f(-1, 4, 4, FAKE, 4, FAKE, 4, FAKE, 4, 0) == gb.GEMM_F32_ERR_DIM
    assert f(5, 9, 8, FAKE, 7, FAKE, 9, FAKE, 9, 0) == gb.GEMM_F32_ERR_LD
    assert f(5, 9, 8, 0, 8, FAKE, 9, FAKE, 9, 0) == gb.GEMM_F32_ERR_NULL
    assert f(5, 9, 8, FAKE + 2, 8, FAKE, 9, FAKE, 9, 0) == gb.GEMM_F32_ERR_ALIGN
    assert f(0, 9, 8, 0, 8, 0, 9, 0, 9, 0) == gb.GEMM_F32_OK
    assert gb.gemm_f32_status_string(gb.GEMM_F32_ERR_SCRATCH) != "unknown status"
    text = open(HEADER).read()
    assert re.search(r"#define GEMM_F32_SCRATCH_BYTES \(\(size_t\)4 << 20\)", text)
    assert gb.GEMM_F32_SCRATCH_BYTES == 4 << 20


def test_every_split_plan_fits_the_static_scratch():
    """A split plan runs at most one 64 x 64 slab per compute unit (256 on a
    whole MI355X), so the 4 MiB scratch holds every one of them."""
    worst = 0
    for M in (16, 64, 65, 100, 128, 200, 256, 300, 640, 700, 1000, 1024):
        for N in (16, 64, 65, 100, 128, 200, 256, 300, 640, 700, 1000, 1024):
            for K in (256, 1024, 4096, 20000, 100000):
                worst = max(worst, gb.gemm_f32_ws_size(M, N, K))
    assert 0 < worst <= gb.GEMM_F32_SCRATCH_BYTES, worst


def test_gpu_tests_plan_what_they_name():
    """The GPU tests that name the plan a shape gets (graph capture per kernel
    family, remainder strips) hold on the host too, so a change of the shape
    rule shows up here before a GPU run."""
    import ast
    src = open(os.path.join(ROOT, "tests", "test_parity.py")).read()
    for var, check in (("GRAPH_PLANS", lambda d, n: d.startswith(n)),
                       ("STRIP", lambda d, n: d.endswith(" " + n))):
        m = re.search(var + r" = (\[.*?\])\n", src, re.S)
        for (M, N, K), name in ast.literal_eval(m.group(1)):
            rc, text = gb.gemm_f32_describe(-1, M, N, K, FAKE, K, FAKE, N, FAKE, N)
            assert rc == gb.GEMM_F32_OK and check(text, name), (var, (M, N, K), text)


def test_poison_lds_flag_reaches_hipcc():
    from dense_fp32_gemm_amd import build
    cmd = build.command("/tmp/x.so", poison_lds=True)
    assert cmd[0] == "hipcc" and "-DGEMM_F32_POISON_LDS" in cmd
    assert "-DGEMM_F32_POISON_LDS" not in build.command("/tmp/x.so")
    assert "--offload-arch=gfx950" in cmd
    src = open(os.path.join(ROOT, "dense_fp32_gemm_amd", "csrc", "gemm_f32.hip")).read()
    assert "#ifdef GEMM_F32_POISON_LDS" in src
    # the normal build is not the poisoned one
    rc, text = gb.gemm_f32_describe(-1, 512, 512, 512, FAKE, 512, FAKE, 512, FAKE, 512)
    assert "poison" not in text, text
