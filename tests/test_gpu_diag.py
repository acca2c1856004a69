"""The measurement aids of include/parallax_diag.h run through the C ABI:
device facts are plausible, the streaming read and the MFMA kernel complete
and leave the sink untouched (its write needs one fixed 64-bit fold)."""
import pytest
import torch

from gpu_common import gpu_available, say

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


def test_device_info():
    from transformer_attention_flash_amd import diag
    info = diag.device_info()
    say(f"diag: device_info {info}")
    assert info["compute_units"] == torch.cuda.get_device_properties(0).multi_processor_count
    assert 500 <= info["max_clock_mhz"] <= 5000
    assert info["bf16_mfma_peak_tflops"] == pytest.approx(
        info["compute_units"] * info["max_clock_mhz"] * 1e6 * 4096 / 1e12)


@pytest.mark.parametrize("nbytes", [16, 16 * 1000, 4 << 20, (64 << 20) + 48])
@pytest.mark.parametrize("nt", [False, True])
def test_stream_read_runs(nbytes, nt):
    from transformer_attention_flash_amd import diag
    say(f"diag: stream_read bytes={nbytes} nontemporal={nt}")
    buf = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    diag.stream_read(buf, nontemporal=nt, sink=sink)
    torch.cuda.synchronize()
    assert sink.item() == 0


def test_mfma_kernel_runs():
    from transformer_attention_flash_amd import diag
    say("diag: mfma_bf16 64 blocks x 100 iterations")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    flops = diag.mfma_bf16(64, 100, sink=sink)
    torch.cuda.synchronize()
    assert flops == 64 * 4 * 8 * 100 * 16384
    assert sink.item() == 0
