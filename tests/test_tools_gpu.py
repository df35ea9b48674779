"""The configuration sweep and the scaling report on the GPU (small sizes)."""
import pytest

from dense_fp32_gemm_amd import binding as gb

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def cuda():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def test_every_configuration_is_resident(cuda):
    for c in range(gb.gemm_f32_num_configs()):
        info = gb.gemm_f32_config_info(c, occupancy=True)
        assert info["blocks_per_cu"] >= 1, gb.gemm_f32_config_name(c)


def test_sweep_checks_every_configuration(cuda):
    from dense_fp32_gemm_amd import sweep
    rows = sweep.sweep_shape(cuda, (300, 270, 77), list(range(gb.gemm_f32_num_configs())),
                             steps=2, warmup=1, log=lambda s: None)
    assert len(rows) == gb.gemm_f32_num_configs() + 1
    assert all(r["ok"] for r in rows), [r for r in rows if not r["ok"]]
    auto = [r for r in rows if r["auto"]]
    assert len(auto) == 1 and auto[0]["config"] == "auto:dma_32x32x32_ksplit4", auto


def test_sweep_times_the_strip_plan(cuda):
    """A strip plan is not any forced configuration: the sweep times it as
    its own candidate."""
    from dense_fp32_gemm_amd import sweep
    cfg = gb.config_names().index("dma_64x64x16_ksplit8_pipe")
    rows = sweep.sweep_shape(cuda, (1025, 1023, 1000), [cfg], steps=2, warmup=1, log=lambda s: None)
    assert [r["config"] for r in rows if r["auto"]] == ["auto:dma_64x64x16_ksplit8_pipe strip_rows=1"], rows
    assert all(r["ok"] for r in rows), rows


def test_report_row(cuda):
    from dense_fp32_gemm_amd import report
    r = report.row_for(cuda, 256, steps=2, warmup=1)
    assert r["check"] == "bit-exact" and r["tflops"] > 0 and r["blocks_per_cu"] >= 1
    assert abs(r["ai"] - 2.0 * 256 ** 3 / (12.0 * 256 * 256)) < 1e-9


def test_device_peak(cuda):
    p = gb.gemm_f32_device_peak(0)
    assert p["compute_units"] == cuda.cuda.get_device_properties(0).multi_processor_count
    assert 1_000_000 <= p["clock_khz"] <= 4_000_000
    assert p["tflops"] == pytest.approx(p["compute_units"] * 256 * p["clock_khz"] * 1e3 / 1e12)


def test_plans_are_sized_from_the_device(cuda):
    """Stream-K runs one worker per compute unit of the current device."""
    cus = cuda.cuda.get_device_properties(0).multi_processor_count
    fake = 0x100000
    rc, text = gb.gemm_f32_describe(-1, 1029, 1025, 1200, fake, 1200, fake, 1025, fake, 1025)
    assert rc == gb.GEMM_F32_OK and f" grid={cus} " in text, text
