"""GPU check of the attainable-peak microbenchmarks (libmla_peaks.so) that
bench.py reports beside the published peaks: each one launches, and each rate
is positive and no higher than the chip's published peak (HBM 8 TB/s, dense
bf16 MFMA 2.5 PFLOP/s; 10 % slack for timing error) -- a rate above it would
mean that the bytes or FLOPs are miscounted or that a cache serves the
rotated rows."""
import pytest
import torch

pytestmark = pytest.mark.gpu

HBM_GBPS, BF16_TFLOPS = 8000.0, 2500.0


@pytest.fixture(scope="module")
def peaks():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sparse_mla_amd import peaks as p
    return p


def test_measured_rates_below_published_peaks(peaks):
    r = peaks.measure()
    print({k: round(v) for k, v in r.items()}, flush=True)
    for k in ("stream_read_GBps", "stream_lds_dma_GBps", "row_gather_GBps"):
        assert 100.0 < r[k] < 1.1 * HBM_GBPS, (k, r[k])
    assert 50.0 < r["mfma_bf16_TFLOPs"] < 1.1 * BF16_TFLOPS, r["mfma_bf16_TFLOPs"]


def test_host_checks_before_launch(peaks):
    sink = torch.zeros(256, dtype=torch.int32, device="cuda")
    cache = torch.zeros(64 * 1152, dtype=torch.uint8, device="cuda")
    rows = torch.zeros(100, dtype=torch.int32, device="cuda")
    with pytest.raises(ValueError):  # fewer rows than num_wg * rows_per_wg
        peaks.row_gather(cache, rows, 4, 32, sink)
    with pytest.raises(RuntimeError):  # rows_per_wg not a multiple of 32: rejected by the library
        peaks.row_gather(cache, rows, 1, 40, sink)
    with pytest.raises(TypeError):
        peaks.mfma_bf16(1, 1, sink)  # the MFMA sink is float32
