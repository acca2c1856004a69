"""GPU parity of the causal-prefill training forward and backward (bf16)
against the fp64 gradient oracle (oracle/grad.py, pinned in
tests/test_oracle_grad_pins.py), on the same rounded inputs.

Tolerance for gradients (bf16 storage, fp32 accumulation): relative L2
<= 1e-2 and max-abs <= 2e-2 * max(1, max |oracle|) per tensor.  The kernels
round p, w, dS and dR to bf16 (relative 2^-9) as matrix-core operands and
round each gradient to bf16 once (relative 2^-9); independent roundings over
a sum give a relative L2 of a few 1e-3, so the bar leaves a ~3x margin while
an indexing or sign mistake gives O(1).
"""
import math

import numpy as np
import pytest
import torch

from gpu_common import TOL, assert_close, errors, gpu_available, host64, say

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

GRAD_TOL = dict(rel_l2=1e-2, max_rel=2e-2)


def _plx():
    import transformer_attention_flash_amd as plx
    return plx


def _inputs(B, Hq, Hkv, T, d, rho, seed=0):
    from transformer_attention_flash_amd import synth
    x = synth.make_prefill(B, Hq, Hkv, T, d, torch.bfloat16, "cuda", seed=seed)
    if not rho:
        x["rho"] = None
    x["dout"] = synth.make_upstream_grad((B, Hq, T, d), torch.bfloat16, "cuda", seed=seed)
    return x


def _check_grad(got, ref, what):
    got = host64(got)
    max_abs, rel = errors(got, ref)
    bar = GRAD_TOL["max_rel"] * max(1.0, float(np.abs(ref).max()))
    say(f"  {what}: max_abs={max_abs:.3e} (bar {bar:.3e}) rel_l2={rel:.3e}")
    assert np.isfinite(got).all(), f"{what}: non-finite"
    assert rel <= GRAD_TOL["rel_l2"], f"{what}: rel_l2 {rel:.3e}"
    assert max_abs <= bar, f"{what}: max_abs {max_abs:.3e} > {bar:.3e}"


def _run(x, scale):
    plx = _plx()
    out, out_sa, lse, rbar = plx.prefill_train(x["q"], x["k"], x["v"], x["rho"], scale=scale)
    grads = plx.prefill_backward(x["q"], x["k"], x["v"], x["rho"], out, out_sa, lse, rbar, x["dout"], scale=scale)
    torch.cuda.synchronize()
    return (out, out_sa, lse, rbar), grads


CASES = [
    # B, Hq, Hkv, T, d, rho
    (1, 2, 1, 100, 64, True),     # G = 2, ragged against every tile size
    (2, 4, 2, 257, 128, True),    # several key blocks and query steps, ragged tail
    (1, 8, 1, 130, 128, True),    # G = 8
    (1, 4, 4, 200, 128, False),   # softmax-only backward, G = 1
    (1, 4, 1, 67, 64, False),     # softmax-only, G = 4
    (1, 1, 1, 1, 64, True),       # one token
    (1, 2, 2, 33, 128, True),     # G = 1, one partial row step
]


@pytest.mark.parametrize("B,Hq,Hkv,T,d,rho", CASES, ids=[f"B{c[0]}_Hq{c[1]}_Hkv{c[2]}_T{c[3]}_d{c[4]}_{'rho' if c[5] else 'sm'}" for c in CASES])
def test_backward_matches_oracle(B, Hq, Hkv, T, d, rho):
    from oracle import grad as ograd
    say(f"backward parity B={B} Hq={Hq} Hkv={Hkv} T={T} d={d} rho={rho}")
    x = _inputs(B, Hq, Hkv, T, d, rho)
    scale = 1.0 / math.sqrt(d)
    _, (dq, dk, dv, drho) = _run(x, scale)
    h = {n: (None if t is None else host64(t)) for n, t in x.items()}
    ref = ograd.grad_expanded(h["q"], h["k"], h["v"], h["rho"], h["dout"], scale)
    _check_grad(dq, ref[0], "dq")
    _check_grad(dk, ref[1], "dk")
    _check_grad(dv, ref[2], "dv")
    if rho:
        _check_grad(drho, ref[3], "drho")
    else:
        assert drho is None


@pytest.mark.parametrize("rho", [True, False])
def test_training_forward_outputs(rho):
    """out equals the inference forward bit for bit; out_sa, lse, rbar match the oracle."""
    from oracle import grad as ograd
    import oracle
    plx = _plx()
    B, Hq, Hkv, T, d = 1, 4, 2, 150, 128
    x = _inputs(B, Hq, Hkv, T, d, rho)
    scale = 1.0 / math.sqrt(d)
    (out, out_sa, lse, rbar), _ = _run(x, scale)
    ref_out = plx.prefill(x["q"], x["k"], x["v"], x["rho"], scale=scale)
    torch.cuda.synchronize()
    assert torch.equal(out, ref_out)
    h = {n: (None if t is None else host64(t)) for n, t in x.items()}
    rows = np.array([[0, hh, t] for hh in range(Hq) for t in range(T)])
    lse_r, rbar_r, osa_r = ograd.forward_stats(h["q"], h["k"], h["v"], h["rho"], scale, rows)
    got_lse = host64(lse).reshape(-1)
    say(f"  lse max err {np.abs(got_lse - lse_r).max():.3e}")
    assert np.abs(got_lse - lse_r).max() <= 5e-3
    if not rho:
        assert rbar is None
    if rho:
        say(f"  rbar max err {np.abs(host64(rbar).reshape(-1) - rbar_r).max():.3e}")
        assert np.abs(host64(rbar).reshape(-1) - rbar_r).max() <= 1e-2
        assert_close(host64(out_sa).reshape(-1, d), osa_r, torch.bfloat16, "out_sa")
        ref = oracle.prefill(h["q"], h["k"], h["v"], h["rho"], scale)
        assert_close(host64(out), ref, torch.bfloat16, "out")
    else:
        assert out_sa is None


def test_backward_deterministic():
    """No atomics anywhere in the training forward or the backward: two runs on
    the same inputs (several key blocks, query steps and a ragged tail) give
    bitwise-equal statistics and gradients."""
    say("backward determinism B=2 Hq=4 Hkv=2 T=257 d=128 rho")
    x = _inputs(2, 4, 2, 257, 128, True, seed=5)
    scale = 1.0 / math.sqrt(128)
    fw1, g1 = _run(x, scale)
    fw2, g2 = _run(x, scale)
    for name, a, b in zip(("out", "out_sa", "lse", "rbar", "dq", "dk", "dv", "drho"), (*fw1, *g1), (*fw2, *g2)):
        assert torch.equal(a, b), f"{name} differs between two identical runs"


def test_autograd_wrapper_matches_entry_points():
    plx = _plx()
    x = _inputs(1, 4, 2, 96, 64, True, seed=3)
    scale = 0.125
    leaves = {n: x[n].clone().requires_grad_(True) for n in ("q", "k", "v", "rho")}
    o = plx.ParallaxAttention.apply(leaves["q"], leaves["k"], leaves["v"], leaves["rho"], scale)
    o.backward(x["dout"])
    _, grads = _run(x, scale)
    for n, g in zip(("q", "k", "v", "rho"), grads):
        assert torch.equal(leaves[n].grad, g), n


@pytest.mark.slow
def test_backward_full_size_sampled_group_and_invariants():
    """B=8, Hq=16, Hkv=8, T=4096, d=128 with a probe: one whole KV-head group
    against the oracle, and over every group the two invariants of the
    gradients: sum_j dv_j = sum over the group's rows of dO (the effective
    weights sum to 1) and sum_j dk_j = 0 (shifting every key leaves o alone)."""
    from oracle import grad as ograd
    B, Hq, Hkv, T, d = 8, 16, 8, 4096, 128
    say("full-size backward B=8 Hq=16 Hkv=8 T=4096 d=128")
    x = _inputs(B, Hq, Hkv, T, d, True)
    scale = 1.0 / math.sqrt(d)
    _, (dq, dk, dv, drho) = _run(x, scale)
    b, g = 5, 3
    G = Hq // Hkv
    hs = slice(g * G, (g + 1) * G)
    h = {n: host64(x[n][b:b + 1, hs] if n in ("q", "rho", "dout") else x[n][b:b + 1, g:g + 1]) for n in x}
    ref = ograd.grad_expanded(h["q"], h["k"], h["v"], h["rho"], h["dout"], scale, groups=[(0, 0)])[(0, 0)]
    _check_grad(dq[b, hs], ref[0], "dq (b=5, kv head 3)")
    _check_grad(dk[b, g], ref[1], "dk (b=5, kv head 3)")
    _check_grad(dv[b, g], ref[2], "dv (b=5, kv head 3)")
    _check_grad(drho[b, hs], ref[3], "drho (b=5, kv head 3)")
    dsum = x["dout"].double().reshape(B, Hkv, G, T, d).sum(dim=(2, 3))
    vsum = dv.double().sum(dim=2)
    rel_v = float((vsum - dsum).norm() / dsum.norm())
    ksum = dk.double().sum(dim=2)
    rel_k = float(ksum.norm() / dk.double().abs().sum(dim=2).norm())
    say(f"  sum_j dv_j vs sum dO: rel {rel_v:.3e}; |sum_j dk_j| / sum_j |dk_j|: {rel_k:.3e}")
    assert rel_v <= 1e-2
    assert rel_k <= 1e-2


def test_backward_persistent_grid_ragged():
    """B=4, Hq=16, Hkv=8, T=1100, d=128 with a probe: 576 dq items and 288
    dk/dv items, more than one workgroup per CU, so both kernels run their
    persistent loops, and T is ragged against both the 64-row and the
    128-key blocks.  The dk/dv items of sequence 3 are the ones the odd
    persistent round takes (key blocks 5-8, walking their rows forwards);
    its KV head 5 and sequence 0's KV head 2 (even rounds, backward walks)
    against the oracle, and the two gradient invariants over every group."""
    from oracle import grad as ograd
    B, Hq, Hkv, T, d = 4, 16, 8, 1100, 128
    say(f"persistent-grid backward B={B} Hq={Hq} Hkv={Hkv} T={T} d={d}")
    x = _inputs(B, Hq, Hkv, T, d, True, seed=5)
    scale = 1.0 / math.sqrt(d)
    _, (dq, dk, dv, drho) = _run(x, scale)
    G = Hq // Hkv
    for b, g in ((3, 5), (0, 2)):
        hs = slice(g * G, (g + 1) * G)
        h = {n: host64(x[n][b:b + 1, hs] if n in ("q", "rho", "dout") else x[n][b:b + 1, g:g + 1]) for n in x}
        ref = ograd.grad_expanded(h["q"], h["k"], h["v"], h["rho"], h["dout"], scale, groups=[(0, 0)])[(0, 0)]
        _check_grad(dq[b, hs], ref[0], f"dq (b={b}, kv head {g})")
        _check_grad(dk[b, g], ref[1], f"dk (b={b}, kv head {g})")
        _check_grad(dv[b, g], ref[2], f"dv (b={b}, kv head {g})")
        _check_grad(drho[b, hs], ref[3], f"drho (b={b}, kv head {g})")
    dsum = x["dout"].double().reshape(B, Hkv, G, T, d).sum(dim=(2, 3))
    rel_v = float((dv.double().sum(dim=2) - dsum).norm() / dsum.norm())
    rel_k = float(dk.double().sum(dim=2).norm() / dk.double().abs().sum(dim=2).norm())
    say(f"  sum_j dv_j vs sum dO: rel {rel_v:.3e}; |sum_j dk_j| / sum_j |dk_j|: {rel_k:.3e}")
    assert rel_v <= 1e-2
    assert rel_k <= 1e-2


def test_backward_beyond_2_31_elements():
    """B=1100, Hq=16, Hkv=8, T=1024, d=128 with a probe: q, rho, dO, o, o^SA,
    dq and drho hold 2.3e9 elements each, so the last sequences sit past
    element 2^31 (64-bit offsets in every backward kernel).  The last
    sequence's last KV-head group against the oracle, plus the two gradient
    invariants on that sequence."""
    from oracle import grad as ograd
    B, Hq, Hkv, T, d = 1100, 16, 8, 1024, 128
    say(f"backward past 2^31 elements: B={B} Hq={Hq} Hkv={Hkv} T={T} d={d} ({B * Hq * T * d} elements per q)")
    x = _inputs(B, Hq, Hkv, T, d, True, seed=3)
    scale = 1.0 / math.sqrt(d)
    _, (dq, dk, dv, drho) = _run(x, scale)
    b, g = B - 1, Hkv - 1
    G = Hq // Hkv
    hs = slice(g * G, (g + 1) * G)
    h = {n: host64(x[n][b:b + 1, hs] if n in ("q", "rho", "dout") else x[n][b:b + 1, g:g + 1]) for n in x}
    ref = ograd.grad_expanded(h["q"], h["k"], h["v"], h["rho"], h["dout"], scale, groups=[(0, 0)])[(0, 0)]
    _check_grad(dq[b, hs], ref[0], f"dq (b={b}, kv head {g})")
    _check_grad(dk[b, g], ref[1], f"dk (b={b}, kv head {g})")
    _check_grad(dv[b, g], ref[2], f"dv (b={b}, kv head {g})")
    _check_grad(drho[b, hs], ref[3], f"drho (b={b}, kv head {g})")
    dsum = x["dout"][b].double().reshape(Hkv, G, T, d).sum(dim=(1, 2))
    vsum = dv[b].double().sum(dim=1)
    rel_v = float((vsum - dsum).norm() / dsum.norm())
    rel_k = float(dk[b].double().sum(dim=1).norm() / dk[b].double().abs().sum(dim=1).norm())
    say(f"  last sequence: sum_j dv_j vs sum dO rel {rel_v:.3e}; |sum_j dk_j| / sum_j |dk_j| {rel_k:.3e}")
    del x, dq, dk, dv, drho
    torch.cuda.empty_cache()
    assert rel_v <= 1e-2
    assert rel_k <= 1e-2
