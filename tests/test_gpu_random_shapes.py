"""GPU parity on seeded random shapes and softmax scales.

The fixed cases elsewhere pick their shapes by hand and use the default
scale 1/sqrt(d).  Here a fixed-seed generator draws batch, head counts, group
size, length, head dimension, dtype, chunk size and a softmax scale away from
1/sqrt(d), so that a kernel that ignored the scale argument, or mishandled an
odd length or head count, fails.  Every output element is compared with the
fp64 oracle.  Short contexts give outputs of size O(1) rather than the O(0.1)
averages of the standard workloads, so the bar is each element's first-order
rounding bound (gpu_common._rows_bound: operand, score and output rounding)
and rel-L2 5e-3.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from gpu_common import assert_within_bound, bound_decode, bound_prefill, errors, gpu_available, host64, say

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

BF, F32 = torch.bfloat16, torch.float32
GROUPS = (1, 2, 4, 8)


def _scale(rng, d):
    # 0.5x .. 2x of 1/sqrt(d): never the default itself.
    return float(rng.choice([0.5, 0.7, 1.3, 2.0])) / math.sqrt(d)


def _prefill_cases(n=40, seed=20261203):
    rng = np.random.default_rng(seed)
    cases = []
    for _ in range(n):
        G = int(rng.choice(GROUPS))
        Hkv = int(rng.integers(1, 3))
        d = int(rng.choice([64, 128]))
        dtype = BF if rng.random() < 0.7 else F32
        T = int(rng.integers(1, 300 if dtype == BF else 160))
        B = int(rng.integers(1, 3))
        rho = bool(rng.random() < 0.8)
        cases.append((B, G * Hkv, Hkv, T, d, dtype, rho, _scale(rng, d)))
    return cases


def _decode_cases(n=40, seed=31):
    rng = np.random.default_rng(seed)
    cases = []
    for _ in range(n):
        G = int(rng.choice(GROUPS))
        Hkv = int(rng.integers(1, 4))
        d = int(rng.choice([64, 128]))
        dtype = BF if rng.random() < 0.75 else F32
        B = int(rng.integers(1, 6))
        ragged = bool(rng.random() < 0.5)
        if ragged:
            lens = [int(x) for x in rng.integers(0, 1500, size=B)]
            if rng.random() < 0.5:
                lens[int(rng.integers(0, B))] = 0  # an empty sequence
        else:
            lens = [int(rng.integers(1, 1500))] * B
        ks = int(rng.choice([0, 0, 32, 64, 160, 512]))
        rho = bool(rng.random() < 0.8)
        cases.append((lens, ragged, G * Hkv, Hkv, d, dtype, ks, rho, _scale(rng, d)))
    return cases


PREFILL = _prefill_cases()
DECODE = _decode_cases()


@pytest.mark.parametrize("case", PREFILL, ids=[f"p{i}" for i in range(len(PREFILL))])
def test_prefill_random_shape(case):
    import transformer_attention_flash_amd as plx
    from transformer_attention_flash_amd import synth
    B, Hq, Hkv, T, d, dtype, rho, scale = case
    say(f"random prefill B={B} Hq={Hq} Hkv={Hkv} T={T} d={d} {dtype} rho={rho} scale={scale:.5f}")
    x = synth.make_prefill(B, Hq, Hkv, T, d, dtype, "cuda", seed=T)
    r = x["rho"] if rho else None
    out = plx.prefill(x["q"], x["k"], x["v"], r, scale=scale)
    torch.cuda.synchronize()
    h = {k: host64(v) for k, v in x.items()}
    r64 = h["rho"] if rho else np.zeros_like(h["q"])
    ref = oracle.prefill(h["q"], h["k"], h["v"], r64, scale)
    assert_within_bound(host64(out), ref, bound_prefill(h["q"], h["k"], h["v"], r64, scale, dtype), "prefill")


@pytest.mark.parametrize("case", DECODE, ids=[f"d{i}" for i in range(len(DECODE))])
def test_decode_random_shape(case):
    import transformer_attention_flash_amd as plx
    from transformer_attention_flash_amd import synth
    lens, ragged, Hq, Hkv, d, dtype, ks, rho, scale = case
    say(f"random decode lens={lens} ragged={ragged} Hq={Hq} Hkv={Hkv} d={d} {dtype} ks={ks} rho={rho} "
        f"scale={scale:.5f}")
    if ragged:
        x = synth.make_decode_ragged(torch.tensor(lens, dtype=torch.int64), Hq, Hkv, d, dtype, "cuda", seed=len(lens))
        kw = dict(cu_seqlens=x["cu_seqlens"], max_ctx=x["max_ctx"], num_kv_heads=Hkv)
        okw = dict(cu_seqlens=x["cu_host"].numpy(), Hkv=Hkv)
    else:
        x = synth.make_decode(len(lens), Hq, Hkv, lens[0], d, dtype, "cuda", seed=lens[0])
        kw, okw = {}, {}
    r = x["rho"] if rho else None
    out = plx.decode(x["q"], x["k"], x["v"], r, scale=scale, keys_per_split=ks, **kw)
    torch.cuda.synchronize()
    q64, rho64, k64, v64 = host64(x["q"]), host64(x["rho"]), host64(x["k"]), host64(x["v"])
    r64 = rho64 if rho else np.zeros_like(q64)
    ref = oracle.decode(q64, r64, k64, v64, scale, **okw)
    bound = bound_decode(q64, r64, k64, v64, scale, dtype, n_merge=1 if ks == 0 else 2, **okw)
    assert_within_bound(host64(out), ref, bound, "decode")


BACKWARD = [
    # B, Hq, Hkv, T, d, rho, scale factor against 1/sqrt(d)
    (1, 6, 3, 91, 64, True, 1.7),
    (2, 2, 1, 150, 128, True, 0.6),
    (1, 8, 2, 45, 64, False, 1.4),
]


@pytest.mark.parametrize("case", BACKWARD, ids=[f"b{i}" for i in range(len(BACKWARD))])
def test_backward_random_scale(case):
    import transformer_attention_flash_amd as plx
    from oracle import grad as ograd
    from transformer_attention_flash_amd import synth
    B, Hq, Hkv, T, d, rho, f = case
    scale = f / math.sqrt(d)
    say(f"random-scale backward B={B} Hq={Hq} Hkv={Hkv} T={T} d={d} rho={rho} scale={scale:.5f}")
    x = synth.make_prefill(B, Hq, Hkv, T, d, BF, "cuda", seed=T)
    r = x["rho"] if rho else None
    dout = synth.make_upstream_grad((B, Hq, T, d), BF, "cuda", seed=T)
    out, out_sa, lse, rbar = plx.prefill_train(x["q"], x["k"], x["v"], r, scale=scale)
    grads = plx.prefill_backward(x["q"], x["k"], x["v"], r, out, out_sa, lse, rbar, dout, scale=scale)
    torch.cuda.synchronize()
    h = {k: host64(v) for k, v in x.items()}
    refs = ograd.grad_expanded(h["q"], h["k"], h["v"], h["rho"] if rho else None, host64(dout), scale)
    names = ("dq", "dk", "dv", "drho")
    for name, got, ref in zip(names, grads, refs):
        if got is None:  # the softmax-only backward has no probe gradient
            assert name == "drho" and not rho
            continue
        g = host64(got)
        max_abs, rel = errors(g, ref)
        bar = 2e-2 * max(1.0, float(np.abs(ref).max()))
        say(f"  {name}: max_abs={max_abs:.3e} (bar {bar:.3e}) rel_l2={rel:.3e}")
        assert np.isfinite(g).all(), name
        assert rel <= 1e-2 and max_abs <= bar, name
