"""The roofline probes return rates in the range the hardware allows."""
import pytest

from lora_shared_kv_amd import skv as B


@pytest.mark.gpu
def test_stream_read_probe(torch_cuda):
    # 1 GiB: four times the infinity cache, so every repetition reads HBM
    buf = torch_cuda.empty(1 << 30, dtype=torch_cuda.uint8, device="cuda")
    gbs = B.skv_probe_stream_read(buf, reps=3)
    assert 500.0 < gbs < 12000.0, gbs


@pytest.mark.gpu
def test_mfma_probe(torch_cuda):
    tflops = B.skv_probe_mfma_bf16()
    assert 100.0 < tflops < 3000.0, tflops


@pytest.mark.gpu
def test_probe_rejects_bad_sizes(torch_cuda):
    buf = torch_cuda.empty(1 << 16, dtype=torch_cuda.uint8, device="cuda")
    with pytest.raises(RuntimeError):
        B.skv_probe_stream_read(buf)  # below the 1 MiB minimum
