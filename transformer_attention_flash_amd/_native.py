"""ctypes view of libparallax.so (include/parallax.h).

Loading the library does not touch the GPU; only the compute entry points
do.  There is no fallback: if the library is missing, every call raises.
"""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libparallax.so")

PLX_OK = 0
PLX_ERR_INVALID_ARGUMENT = 1
PLX_ERR_UNSUPPORTED = 2
PLX_ERR_WORKSPACE_TOO_SMALL = 3
PLX_ERR_HIP = 4

PLX_DTYPE_F32 = 0
PLX_DTYPE_BF16 = 1

# Bytes of the per-device scratch of parallax_fwd_decode_noalloc
# (PLX_DECODE_NOALLOC_SCRATCH_BYTES in include/parallax.h).
DECODE_NOALLOC_SCRATCH_BYTES = 16 << 20

# Every symbol include/parallax.h declares.
EXPORTS = (
    "parallax_fwd_prefill",
    "parallax_fwd_prefill_train",
    "parallax_bwd_prefill_workspace_size",
    "parallax_bwd_prefill",
    "parallax_qkvr_projection",
    "parallax_fwd_decode",
    "parallax_fwd_decode_workspace_size",
    "parallax_fwd_decode_auto_split",
    "parallax_fwd_decode_chunked",
    "parallax_fwd_decode_chunked_workspace_size",
    "parallax_fwd_decode_noalloc",
    "parallax_status_string",
    "parallax_diag_device_info",
    "parallax_diag_stream_read",
    "parallax_diag_mfma_bf16",
)

_lib = None


class ParallaxError(RuntimeError):
    """A non-OK status from libparallax."""

    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


def load():
    """Load libparallax.so once and declare its signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is not built; run `python -m transformer_attention_flash_amd.build` "
            "(there is no non-HIP fallback)")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
    lib.parallax_fwd_prefill.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, f32, ctypes.c_int, vp]
    lib.parallax_fwd_prefill.restype = ctypes.c_int
    lib.parallax_fwd_prefill_train.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, f32,
                                               ctypes.c_int, vp]
    lib.parallax_fwd_prefill_train.restype = ctypes.c_int
    lib.parallax_bwd_prefill_workspace_size.argtypes = [i32, i32, i32]
    lib.parallax_bwd_prefill_workspace_size.restype = ctypes.c_size_t
    lib.parallax_bwd_prefill.argtypes = [vp] * 13 + [i32, i32, i32, i32, i32, f32, ctypes.c_int, vp,
                                                     ctypes.c_size_t, vp]
    lib.parallax_bwd_prefill.restype = ctypes.c_int
    lib.parallax_qkvr_projection.argtypes = [vp] * 6 + [i32] * 6 + [ctypes.c_int, vp]
    lib.parallax_qkvr_projection.restype = ctypes.c_int
    lib.parallax_fwd_decode_workspace_size.argtypes = [i32, i32, i32, i32, i64, ctypes.c_int]
    lib.parallax_fwd_decode_workspace_size.restype = ctypes.c_size_t
    lib.parallax_fwd_decode.argtypes = [vp, vp, vp, vp, vp, i64, vp, i32, i32, i32, i32, f32, ctypes.c_int,
                                        vp, ctypes.c_size_t, vp]
    lib.parallax_fwd_decode.restype = ctypes.c_int
    lib.parallax_fwd_decode_chunked_workspace_size.argtypes = [i32, i32, i32, i32, i64, ctypes.c_int, i32]
    lib.parallax_fwd_decode_chunked_workspace_size.restype = ctypes.c_size_t
    lib.parallax_fwd_decode_chunked.argtypes = [vp, vp, vp, vp, vp, i64, vp, i32, i32, i32, i32, f32,
                                                ctypes.c_int, i32, vp, ctypes.c_size_t, vp]
    lib.parallax_fwd_decode_chunked.restype = ctypes.c_int
    lib.parallax_fwd_decode_noalloc.argtypes = [vp, vp, vp, vp, vp, i64, vp, i32, i32, i32, i32, f32,
                                                ctypes.c_int, vp]
    lib.parallax_fwd_decode_noalloc.restype = ctypes.c_int
    lib.parallax_fwd_decode_auto_split.argtypes = [i32, i32, i32, i32, i64]
    lib.parallax_fwd_decode_auto_split.restype = i32
    lib.parallax_status_string.argtypes = [ctypes.c_int]
    lib.parallax_status_string.restype = ctypes.c_char_p
    lib.parallax_diag_device_info.argtypes = [i32, ctypes.POINTER(i32), ctypes.POINTER(i32)]
    lib.parallax_diag_device_info.restype = ctypes.c_int
    lib.parallax_diag_stream_read.argtypes = [vp, ctypes.c_size_t, i32, vp, vp]
    lib.parallax_diag_stream_read.restype = ctypes.c_int
    lib.parallax_diag_mfma_bf16.argtypes = [vp, i32, i32, vp]
    lib.parallax_diag_mfma_bf16.restype = ctypes.c_int
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().parallax_status_string(int(status)).decode()


def check(status: int, where: str) -> None:
    if status != PLX_OK:
        raise ParallaxError(status, where)
