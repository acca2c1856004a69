"""Python side of the measurement aids in include/parallax_diag.h: device
facts, a plain streaming-read kernel and a bf16 MFMA throughput kernel.
Argument marshalling only; the kernels are in libparallax.so."""
from __future__ import annotations

import ctypes
from typing import Optional

import torch

from . import _native as N
from .api import _stream

MFMA_FLOP = 2 * 16 * 16 * 32      # one v_mfma_f32_16x16x32_bf16
BF16_FLOP_PER_CLOCK_PER_CU = 4096  # 4 SIMDs x one such MFMA per 16 cycles


def device_info(device: Optional[int] = None) -> dict:
    """Compute units and maximum engine clock as the HIP runtime reports them,
    and the dense bf16 MFMA peak they imply."""
    if device is None:
        device = torch.cuda.current_device()
    cu, clk = ctypes.c_int32(), ctypes.c_int32()
    N.check(N.load().parallax_diag_device_info(int(device), ctypes.byref(cu), ctypes.byref(clk)),
            "parallax_diag_device_info")
    return {"compute_units": cu.value, "max_clock_mhz": clk.value / 1e3,
            "bf16_mfma_peak_tflops": cu.value * clk.value * 1e3 * BF16_FLOP_PER_CLOCK_PER_CU / 1e12}


def _sink(sink: Optional[torch.Tensor], device) -> torch.Tensor:
    if sink is None:
        sink = torch.zeros(1, dtype=torch.int32, device=device)
    if not sink.is_cuda or sink.numel() * sink.element_size() < 4:
        raise ValueError("sink must be a GPU tensor of at least 4 bytes")
    return sink


def stream_read(buf: torch.Tensor, *, nontemporal: bool = True, sink: Optional[torch.Tensor] = None,
                stream=None) -> None:
    """Read every byte of `buf` once (contiguous, a multiple of 16 bytes)."""
    if not buf.is_cuda or not buf.is_contiguous():
        raise ValueError("buf must be a contiguous GPU tensor")
    sink = _sink(sink, buf.device)
    N.check(N.load().parallax_diag_stream_read(buf.data_ptr(), buf.numel() * buf.element_size(),
                                               1 if nontemporal else 0, sink.data_ptr(), _stream(stream)),
            "parallax_diag_stream_read")


def mfma_bf16(n_blocks: int, iterations: int, *, sink: Optional[torch.Tensor] = None, stream=None) -> int:
    """Launch the MFMA throughput kernel; returns the flops it performs."""
    sink = _sink(sink, torch.device("cuda", torch.cuda.current_device()))
    N.check(N.load().parallax_diag_mfma_bf16(sink.data_ptr(), int(n_blocks), int(iterations), _stream(stream)),
            "parallax_diag_mfma_bf16")
    return int(n_blocks) * 4 * 8 * int(iterations) * MFMA_FLOP
