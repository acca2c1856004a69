"""parallax_fwd_decode_noalloc (the decode entry point that allocates
nothing: its split partials live in the library's own per-device scratch)
against parallax_fwd_decode with a caller workspace, through the C ABI.

Two calls in a row, the second smaller, each with more than one chunk per
sequence so that the scratch is written and read by the merge kernel: the
outputs must equal parallax_fwd_decode's bit for bit (same kernels, same
chunking), and both must meet the fp64 oracle at the bf16 bar.  The second
call also shows that what the first left in the scratch does not leak into
it.
"""
import numpy as np
import pytest
import torch

import oracle
import transformer_attention_flash_amd as plx
from transformer_attention_flash_amd import _native as N
from transformer_attention_flash_amd import synth

from gpu_common import assert_close, host64, say

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _compare(x, ragged=None):
    kw = {}
    if ragged is not None:
        kw = dict(cu_seqlens=x["cu_seqlens"], max_ctx=x["max_ctx"], num_kv_heads=ragged)
    B, Hq, d = x["q"].shape
    Hkv = ragged if ragged is not None else x["k"].shape[1]
    L = x["max_ctx"] if ragged is not None else x["k"].shape[2]
    ws = plx.decode_workspace_size(B, Hq, Hkv, d, L)
    assert 0 < ws <= N.DECODE_NOALLOC_SCRATCH_BYTES, "the case must split and fit the scratch"
    want = plx.decode(x["q"], x["k"], x["v"], x["rho"], **kw)
    out = torch.full_like(x["q"], float("nan"))
    got = plx.decode_noalloc(x["q"], x["k"], x["v"], x["rho"], out=out, **kw)
    torch.cuda.synchronize()
    assert got.data_ptr() == out.data_ptr()
    assert torch.equal(got, want), "noalloc decode differs from parallax_fwd_decode"
    h = {n: host64(x[n]) for n in ("q", "k", "v", "rho")}
    if ragged is None:
        ref = oracle.decode(h["q"], h["rho"], h["k"], h["v"], 1 / np.sqrt(d))
    else:
        ref = oracle.decode(h["q"], h["rho"], h["k"], h["v"], 1 / np.sqrt(d), cu_seqlens=x["cu_host"].numpy(),
                            Hkv=ragged)
    assert_close(host64(got), ref, torch.bfloat16, f"noalloc decode B={B} Hq={Hq} Hkv={Hkv} L={L} d={d}")


def test_noalloc_decode_two_calls_second_smaller():
    say("noalloc decode: call 1, contiguous B=3 Hq=16 Hkv=8 L=8192 d=128")
    _compare(synth.make_decode(3, 16, 8, 8192, 128, torch.bfloat16, DEV, seed=31))
    say("noalloc decode: call 2, ragged B=2 Hq=8 Hkv=4 lengths 1500, 2900 d=64")
    lengths = torch.tensor([1500, 2900], dtype=torch.int64)
    _compare(synth.make_decode_ragged(lengths, 8, 4, 64, torch.bfloat16, DEV, seed=32), ragged=4)


def test_noalloc_decode_single_chunk_uses_no_scratch():
    """A call that needs no workspace (one chunk per sequence) takes the same
    path as parallax_fwd_decode."""
    say("noalloc decode: single chunk B=64 Hq=16 Hkv=8 L=1024 d=128")
    x = synth.make_decode(64, 16, 8, 1024, 128, torch.bfloat16, DEV, seed=33)
    assert plx.decode_workspace_size(64, 16, 8, 128, 1024) == 0
    want = plx.decode(x["q"], x["k"], x["v"], x["rho"])
    got = plx.decode_noalloc(x["q"], x["k"], x["v"], x["rho"])
    torch.cuda.synchronize()
    assert torch.equal(got, want)
