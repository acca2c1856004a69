"""GPU parity of the fused q/k/v/probe projection (bf16) against the fp64
oracle (oracle/projection.py) on the same rounded inputs.

Bar, per element: |got - ref| <= 2^-8 |ref| + 1e-3 rms(ref).  The kernel
accumulates in fp32 and rounds each output once to bf16: round-to-nearest
with 8 significant bits errs by at most half an ulp, 2^-8 of the value's
power-of-two floor, so at most 2^-8 |ref|; the absolute floor covers the
fp32 accumulation over d_model terms for outputs near zero.
"""
import numpy as np
import pytest
import torch

from gpu_common import gpu_available, host64, say

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


def _check(got, ref, what):
    got = host64(got)
    err = np.abs(got - ref)
    bound = 2.0 ** -8 * np.abs(ref) + 1e-3 * float(np.sqrt((ref ** 2).mean()))
    worst = float((err / bound).max()) if err.size else 0.0
    rel = float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30))
    say(f"  {what}: max_abs={float(err.max()):.3e} rel_l2={rel:.3e} worst err/bound={worst:.3f}")
    assert np.isfinite(got).all()
    assert worst <= 1.0, f"{what}: error above the bar"


CASES = [
    # B, T, d_model, Hq, Hkv, d
    (2, 67, 128, 4, 2, 64),      # ragged token count, 128-feature blocks spanning two heads
    (1, 300, 256, 2, 1, 128),
    (3, 129, 192, 8, 8, 64),     # G = 1, d_model not a power of two
    (1, 1, 64, 1, 1, 64),        # one token
]


@pytest.mark.parametrize("B,T,dm,Hq,Hkv,d", CASES, ids=[f"B{c[0]}_T{c[1]}_dm{c[2]}_Hq{c[3]}_Hkv{c[4]}_d{c[5]}" for c in CASES])
def test_projection_matches_oracle(B, T, dm, Hq, Hkv, d):
    import transformer_attention_flash_amd as plx
    from transformer_attention_flash_amd import synth
    from oracle import projection as oproj
    say(f"projection parity B={B} T={T} d_model={dm} Hq={Hq} Hkv={Hkv} d={d}")
    x, w = synth.make_projection(B, T, dm, Hq, Hkv, d, torch.bfloat16, "cuda")
    outs = plx.qkvr_projection(x, w, Hq, Hkv, d)
    torch.cuda.synchronize()
    refs = oproj.project(host64(x), host64(w), Hq, Hkv, d)
    for name, got, ref in zip(("q", "k", "v", "rho"), outs, refs):
        _check(got, ref, name)


def test_projection_deterministic():
    """Each output element is one block's fp32 sum in a fixed order: two calls
    (several feature and token blocks, a ragged token tail) are bitwise equal."""
    import transformer_attention_flash_amd as plx
    from transformer_attention_flash_amd import synth
    say("projection determinism B=2 T=600 d_model=256 Hq=4 Hkv=2 d=128")
    x, w = synth.make_projection(2, 600, 256, 4, 2, 128, torch.bfloat16, "cuda", seed=3)
    a = plx.qkvr_projection(x, w, 4, 2, 128)
    b = plx.qkvr_projection(x, w, 4, 2, 128)
    torch.cuda.synchronize()
    for name, u, v in zip(("q", "k", "v", "rho"), a, b):
        assert torch.equal(u, v), f"{name} differs between two identical calls"


def test_projection_full_size_sampled_tokens():
    """The prefill workload's projection (B=8, T=4096, d_model=2048, Hq=16,
    Hkv=8, d=128): 96 sampled tokens against the oracle, every output
    feature."""
    import transformer_attention_flash_amd as plx
    from transformer_attention_flash_amd import synth
    from oracle import projection as oproj
    B, T, dm, Hq, Hkv, d = 8, 4096, 2048, 16, 8, 128
    say("projection full size B=8 T=4096 d_model=2048 Hq=16 Hkv=8 d=128")
    x, w = synth.make_projection(B, T, dm, Hq, Hkv, d, torch.bfloat16, "cuda")
    outs = plx.qkvr_projection(x, w, Hq, Hkv, d)
    torch.cuda.synchronize()
    rng = np.random.default_rng(7)
    bs = rng.integers(0, B, 96)
    ts = rng.integers(0, T, 96)
    ts[:4] = [0, 4095, 127, 128]
    xs = host64(x[torch.tensor(bs), torch.tensor(ts)])[:, None, :]  # [96, 1, dm] as 96 one-token batches
    refs = oproj.project(xs, host64(w), Hq, Hkv, d)
    for name, got, ref in zip(("q", "k", "v", "rho"), outs, refs):
        g = got[torch.tensor(bs), :, torch.tensor(ts)]               # [96, H, d]
        _check(g[:, :, None, :], ref, name)


def test_projection_beyond_2_31_elements():
    """B=2, T=540000 tokens, d_model=2048, Hq=16, Hkv=8, d=128: q and rho hold
    2.2e9 elements each, so the last tokens' outputs sit past element 2^31
    (64-bit output offsets); sampled tokens at both ends against the oracle."""
    import transformer_attention_flash_amd as plx
    from transformer_attention_flash_amd import synth
    from oracle import projection as oproj
    B, T, dm, Hq, Hkv, d = 2, 540000, 2048, 16, 8, 128
    say(f"projection past 2^31 elements: B={B} T={T} ({B * T * Hq * d} elements per q)")
    x, w = synth.make_projection(B, T, dm, Hq, Hkv, d, torch.bfloat16, "cuda")
    outs = plx.qkvr_projection(x, w, Hq, Hkv, d)
    torch.cuda.synchronize()
    bs = np.array([0, 0, 1, 1, 1, 1])
    ts = np.array([0, T - 1, 0, 255, T - 256, T - 1])
    xs = host64(x[torch.tensor(bs), torch.tensor(ts)])[:, None, :]
    refs = oproj.project(xs, host64(w), Hq, Hkv, d)
    for name, got, ref in zip(("q", "k", "v", "rho"), outs, refs):
        g = got[torch.tensor(bs), :, torch.tensor(ts)]
        _check(g[:, :, None, :], ref, name)
    del x, w, outs
    torch.cuda.empty_cache()
