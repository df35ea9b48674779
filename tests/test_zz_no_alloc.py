"""gemm_f32_ws_noalloc: split-K through the library's static scratch (no
allocation) must give exactly what gemm_f32_ws gives with a caller's
workspace, on consecutive calls that reuse the scratch, the second smaller."""
import sys

import numpy as np
import pytest

import oracle
from dense_fp32_gemm_amd import binding as gb
from dense_fp32_gemm_amd import inputs
from checks import assert_bit_exact

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu


def say(*msg):
    print("[no-alloc]", *msg, file=sys.__stderr__, flush=True)


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def run_both(dev, A, B):
    """(C from gemm_f32_ws_noalloc, C from gemm_f32_ws), both NaN-filled first."""
    M, K = A.shape
    N = B.shape[1]
    need = gb.gemm_f32_ws_size(M, N, K)
    dA = torch.from_numpy(A).to(dev)
    dB = torch.from_numpy(B).to(dev)
    c_static = torch.full((M, N), float("nan"), device=dev)
    c_ws = torch.full((M, N), float("nan"), device=dev)
    ws = torch.full((max(1, need // 4),), float("nan"), device=dev)
    s = torch.cuda.current_stream().cuda_stream
    say(f"gemm_f32_ws_noalloc M={M} N={N} K={K} (split plan needs {need} bytes)")
    rc = gb.gemm_f32_ws_noalloc(M, N, K, dA.data_ptr(), K, dB.data_ptr(), N, c_static.data_ptr(), N, s)
    assert rc == gb.GEMM_F32_OK, gb.gemm_f32_status_string(rc)
    torch.cuda.synchronize()
    say(f"gemm_f32_ws M={M} N={N} K={K}")
    rc = gb.gemm_f32_ws(M, N, K, dA.data_ptr(), K, dB.data_ptr(), N, c_ws.data_ptr(), N,
                        ws.data_ptr(), need, s)
    assert rc == gb.GEMM_F32_OK, gb.gemm_f32_status_string(rc)
    torch.cuda.synchronize()
    return c_static.cpu().numpy(), c_ws.cpu().numpy(), need


def test_noalloc_matches_the_workspace_entry_point_on_consecutive_calls(dev):
    # a larger split plan, then a smaller one: the second reuses scratch that
    # still holds the first call's partial products
    for kind, shape in (("quarter", (200, 200, 20000)), ("quarter", (130, 70, 5000)),
                        ("uniform", (600, 600, 4096)), ("uniform", (64, 300, 3000))):
        A, B = (inputs.quarter_step if kind == "quarter" else inputs.uniform)(*shape)
        got, want, need = run_both(dev, A, B)
        assert 0 < need <= gb.GEMM_F32_SCRATCH_BYTES, (shape, need)
        assert_bit_exact(got, want, f"{shape} {kind}: no-alloc against workspace")
        if kind == "quarter":
            assert_bit_exact(got, oracle.gemm(A, B), f"{shape} against the oracle")


def test_noalloc_unsplit_shapes_run_the_plain_path(dev):
    for shape in ((1025, 1023, 1000), (17, 33, 65), (1000, 1000, 300)):
        A, B = inputs.quarter_step(*shape)
        got, want, need = run_both(dev, A, B)
        assert need == 0
        assert_bit_exact(got, want, f"{shape}")
        assert_bit_exact(got, oracle.gemm(A, B), f"{shape} against the oracle")
