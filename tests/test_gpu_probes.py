"""The roofline probes return rates in the range the hardware allows, and check
their arguments before any device call."""
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
def test_mfma_probe_on_operand_data(torch_cuda):
    g = torch_cuda.Generator(device="cuda")
    g.manual_seed(7)
    operands = torch_cuda.randn(8192, generator=g, device="cuda").to(torch_cuda.bfloat16)
    tflops = B.skv_probe_mfma_bf16_data(operands)
    assert 100.0 < tflops < 3000.0, tflops


def test_mfma_data_probe_checks_arguments():
    with pytest.raises(B.SkvError) as e:
        B.skv_probe_mfma_bf16_data(0, kind="host")
    assert e.value.code == "ARG"
    with pytest.raises(B.SkvError) as e:
        B.skv_probe_mfma_bf16_data(1 << 40, kind="host")
    assert e.value.code == "UNSUPPORTED"


@pytest.mark.gpu
def test_probe_rejects_bad_sizes(torch_cuda):
    buf = torch_cuda.empty(1 << 16, dtype=torch_cuda.uint8, device="cuda")
    with pytest.raises(RuntimeError):
        B.skv_probe_stream_read(buf)  # below the 1 MiB minimum


@pytest.mark.gpu
def test_launch_pattern_probe(torch_cuda):
    # four 32 MiB layers (128 MiB per step) with a 128-workgroup launch after each
    layer = 32 << 20
    buf = torch_cuda.empty(4 * layer, dtype=torch_cuda.uint8, device="cuda")
    pat, stream = B.skv_probe_launch_pattern(buf, layer, 4, steps=5, tail_blocks=128)
    assert 0.0 < stream and 0.0 < pat < 100.0, (pat, stream)
    # the streaming reads alone cannot beat the HBM rate by much, nor can a
    # step with the small launches take less than its reads by much
    assert 4 * layer / (stream * 1e-3) / 1e9 < 12000.0
    assert pat > 0.9 * stream, (pat, stream)


def test_launch_pattern_probe_checks_arguments():
    # argument checks run before any device call; the CPU-only build then
    # reports UNSUPPORTED for a well-formed call
    addr = 1 << 40
    for layer_bytes, layers, steps, tail in ((1 << 16, 4, 5, 128), ((1 << 20) + 8, 4, 5, 128),
                                             (1 << 20, 0, 5, 128), (1 << 20, 4, 0, 128), (1 << 20, 4, 5, 0),
                                             (1 << 20, 2000, 5, 128), (1 << 20, 4, 5000, 128)):
        with pytest.raises(B.SkvError) as e:
            B.skv_probe_launch_pattern(addr, layer_bytes, layers, steps, tail, kind="host")
        assert e.value.code == "ARG", (layer_bytes, layers, steps, tail)
    with pytest.raises(B.SkvError) as e:
        B.skv_probe_launch_pattern(addr, 1 << 20, 4, 5, 128, kind="host")
    assert e.value.code == "UNSUPPORTED"
