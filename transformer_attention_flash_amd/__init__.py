"""Parallax attention on AMD MI355X (gfx950): forward (prefill, decode) and
the causal-prefill backward.

The computation lives in libparallax.so (hand-written HIP kernels behind the
C ABI of include/parallax.h); this package binds it with ctypes and offers
seeded synthetic inputs.  PyTorch supplies device memory and streams only.
"""
from ._native import EXPORTS, LIB_PATH, ParallaxError, load as load_library
from .api import (ParallaxAttention, decode, decode_auto_split, decode_noalloc, decode_workspace_size,
                  parallax_bwd_prefill, parallax_fwd_decode, parallax_fwd_decode_auto_split,
                  parallax_fwd_decode_chunked, parallax_fwd_decode_noalloc, parallax_fwd_decode_workspace_size,
                  parallax_fwd_prefill, parallax_fwd_prefill_train, parallax_qkvr_projection, prefill,
                  prefill_backward, prefill_train, qkvr_projection)

__all__ = ["prefill", "prefill_train", "prefill_backward", "ParallaxAttention", "qkvr_projection", "decode",
           "decode_workspace_size", "decode_auto_split", "parallax_fwd_prefill", "parallax_fwd_prefill_train",
           "parallax_bwd_prefill", "parallax_qkvr_projection", "parallax_fwd_decode",
           "parallax_fwd_decode_workspace_size", "parallax_fwd_decode_auto_split", "parallax_fwd_decode_chunked",
           "parallax_fwd_decode_noalloc", "decode_noalloc",
           "ParallaxError", "LIB_PATH", "EXPORTS", "load_library"]
