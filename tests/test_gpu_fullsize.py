"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times (library-chosen chunking), against the fp64 oracle on EVERY
output row.

The oracle reads back the same rounded tensors from the device (converted to
fp64 on the device, which is exact, and copied to the host).  The two caches
too large for host memory at once (256 x 32768 keys, 34 GB; the ragged batch,
137 GB) are streamed through the oracle a group of whole sequences at a time
through one pinned staging buffer.

Besides the expanded form (every row), the explicit-covariance form of the
oracle runs on a seeded sample of at least 64 rows per workload, always
including the first and last sequence or position and, for the ragged batch,
the shortest and longest sequences.  The two oracle forms must agree to 1e-12
relative, and the GPU must meet the same bar against either.
"""
import time

import numpy as np
import pytest
import torch

import oracle
import transformer_attention_flash_amd as plx
from transformer_attention_flash_amd import synth

from gpu_common import assert_close, host64, say

pytestmark = pytest.mark.gpu
DEV = "cuda"
STAGE_BYTES = 1 << 30  # pinned fp64 staging for the streamed caches


@pytest.fixture(autouse=True)
def _free_memory():
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _pick(n, k, rng, must=()):
    picks = set(int(m) for m in must if 0 <= m < n)
    while len(picks) < min(k, n):
        picks.add(int(rng.integers(0, n)))
    return sorted(picks)


class _Stage:
    """Pinned host buffer that device tensors are converted into as fp64."""

    def __init__(self, nbytes=STAGE_BYTES):
        self.buf = torch.empty(nbytes // 8, dtype=torch.float64, pin_memory=True)

    def fetch(self, t: torch.Tensor, slot: int, nslots: int) -> np.ndarray:
        n = t.numel()
        per = self.buf.numel() // nslots
        assert n <= per, f"{n} elements exceed a staging slot of {per}"
        view = self.buf[slot * per:slot * per + n]
        view.copy_(t.reshape(-1).to(torch.float64))
        return view.numpy()


def _forms_agree(expanded, explicit, what):
    """The oracle's two forms agree to 1e-12 relative (max-abs over the rows,
    relative to the largest output)."""
    scale = max(float(np.abs(expanded).max()), 1e-300)
    rel = float(np.abs(expanded - explicit).max()) / scale
    say(f"  {what}: explicit vs expanded oracle, {explicit.shape[0]} rows, max rel diff {rel:.2e}")
    assert rel <= 1e-12, f"{what}: the oracle's explicit and expanded forms differ by {rel:.2e}"


@pytest.mark.parametrize("name,ks", [("decode_bf16_b64_hq16_hkv8_l4096_d128", 0),
                                     ("decode_bf16_b64_hq16_hkv8_l4096_d128", 256),
                                     ("decode_bf16_b2048_hq16_hkv8_l128_d128", 0)])
def test_decode_full_size_every_row(name, ks):
    """ks = 0: the library's chunking (one chunk per sequence here); ks = 256:
    16 chunks per sequence through parallax_fwd_decode_chunked, so the merge
    kernel runs at full size."""
    w = synth.WORKLOADS[name]
    say(f"full-size {name}, keys_per_split={ks or 'library'}")
    x = synth.make_workload(w, DEV)
    out = plx.decode(x["q"], x["k"], x["v"], x["rho"], keys_per_split=ks)
    out2 = plx.decode(x["q"], x["k"], x["v"], x["rho"], keys_per_split=ks)
    torch.cuda.synchronize()
    assert torch.equal(out, out2), "repeated call differs"
    h = {n: host64(x[n]) for n in ("q", "k", "v", "rho")}
    tau = 1 / np.sqrt(w.d)
    ref = oracle.decode(h["q"], h["rho"], h["k"], h["v"], tau)
    got = host64(out)
    assert_close(got, ref, w.dtype, f"{name}: all {w.B} sequences x {w.Hq} heads")
    if ks == 0:
        rng = np.random.default_rng(3)
        rows = np.array([(b, hh) for b in _pick(w.B, 8, rng, must=(0, w.B - 1)) for hh in range(w.Hq)])
        exp = oracle.decode(h["q"], h["rho"], h["k"], h["v"], tau, form=oracle.EXPLICIT, rows=rows)
        _forms_agree(ref[rows[:, 0], rows[:, 1]], exp, name)
        assert_close(got[rows[:, 0], rows[:, 1]], exp, w.dtype, f"{name}: {len(rows)} rows vs explicit form")


def test_decode_long_context_every_row_streamed():
    """256 sequences x 32768 keys (34 GB of K/V): every row, one sequence at a
    time through the oracle."""
    name = "decode_bf16_b256_hq16_hkv8_l32768_d128"
    w = synth.WORKLOADS[name]
    say(f"full-size {name}")
    x = synth.make_workload(w, DEV)
    out = plx.decode(x["q"], x["k"], x["v"], x["rho"])
    torch.cuda.synchronize()
    got = host64(out)
    q, rho = host64(x["q"]), host64(x["rho"])
    tau = 1 / np.sqrt(w.d)
    ref = np.zeros_like(got)
    stage = _Stage()
    rng = np.random.default_rng(4)
    explicit_seqs = _pick(w.B, 4, rng, must=(0, w.B - 1))
    exp_rows, exp_ref, exp_got = [], [], []
    t0 = time.time()
    for b in range(w.B):
        kb = stage.fetch(x["k"][b], 0, 2).reshape(1, w.Hkv, w.L, w.d)
        vb = stage.fetch(x["v"][b], 1, 2).reshape(1, w.Hkv, w.L, w.d)
        ref[b] = oracle.decode(q[b:b + 1], rho[b:b + 1], kb, vb, tau)[0]
        if b in explicit_seqs:
            exp_ref.append(ref[b])
            exp_rows.append(oracle.decode(q[b:b + 1], rho[b:b + 1], kb, vb, tau, form=oracle.EXPLICIT)[0])
            exp_got.append(got[b])
        if b % 64 == 63:
            say(f"  oracle through sequence {b + 1} of {w.B} ({time.time() - t0:.0f} s)")
    assert_close(got, ref, w.dtype, f"{name}: all {w.B} sequences x {w.Hq} heads")
    exp = np.concatenate(exp_rows)
    _forms_agree(np.concatenate(exp_ref), exp, name)
    assert_close(np.concatenate(exp_got), exp, w.dtype, f"{name}: {exp.shape[0]} rows vs explicit form")


def test_ragged_decode_every_row_streamed():
    """The ragged batch (2048 sequences of 128..32768 keys, 137 GB of K/V):
    every row, groups of whole sequences at a time through the oracle."""
    name = "decode_ragged_bf16_b2048_hq32_hkv16_d64_l128to32768"
    w = synth.WORKLOADS[name]
    say(f"full-size {name}")
    x = synth.make_workload(w, DEV)
    cu = x["cu_host"].numpy()
    lens = np.diff(cu)
    say(f"  sum of lengths {int(cu[-1])}, KV bytes {4 * w.Hkv * w.d * int(cu[-1]) / 1e9:.1f} GB")
    out = plx.decode(x["q"], x["k"], x["v"], x["rho"], cu_seqlens=x["cu_seqlens"], max_ctx=x["max_ctx"],
                     num_kv_heads=w.Hkv)
    torch.cuda.synchronize()
    got = host64(out)
    q, rho = host64(x["q"]), host64(x["rho"])
    tau = 1 / np.sqrt(w.d)
    per_tok = w.Hkv * w.d
    stage = _Stage()
    slot_tokens = stage.buf.numel() // 2 // per_tok
    ref = np.zeros_like(got)
    rng = np.random.default_rng(5)
    explicit_seqs = set(_pick(w.B, 4, rng, must=(0, w.B - 1, int(lens.argmin()), int(lens.argmax()))))
    exp_rows, exp_ref, exp_got = [], [], []
    t0 = time.time()
    b0 = 0
    while b0 < w.B:
        b1 = b0 + 1
        while b1 < w.B and cu[b1 + 1] - cu[b0] <= slot_tokens:
            b1 += 1
        s0, s1 = int(cu[b0]) * per_tok, int(cu[b1]) * per_tok
        kb = stage.fetch(x["k"][s0:s1], 0, 2)
        vb = stage.fetch(x["v"][s0:s1], 1, 2)
        sub_cu = cu[b0:b1 + 1] - cu[b0]
        ref[b0:b1] = oracle.decode(q[b0:b1], rho[b0:b1], kb, vb, tau, cu_seqlens=sub_cu, Hkv=w.Hkv)
        for b in sorted(explicit_seqs & set(range(b0, b1))):
            one = np.array([0, lens[b]])
            o = int(cu[b] - cu[b0]) * per_tok
            kk, vv = kb[o:o + lens[b] * per_tok], vb[o:o + lens[b] * per_tok]
            exp_rows.append(oracle.decode(q[b:b + 1], rho[b:b + 1], kk, vv, tau, cu_seqlens=one, Hkv=w.Hkv,
                                          form=oracle.EXPLICIT)[0])
            exp_ref.append(ref[b])
            exp_got.append(got[b])
        if b1 // 512 > b0 // 512:
            say(f"  oracle through sequence {b1} of {w.B} ({time.time() - t0:.0f} s)")
        b0 = b1
    assert_close(got, ref, w.dtype, f"{name}: all {w.B} sequences x {w.Hq} heads")
    exp = np.concatenate(exp_rows)
    _forms_agree(np.concatenate(exp_ref), exp, name)
    assert_close(np.concatenate(exp_got), exp, w.dtype,
                 f"{name}: {exp.shape[0]} rows (lengths {sorted(lens[sorted(explicit_seqs)].tolist())}) vs explicit")


def test_prefill_full_size_every_row():
    name = "prefill_bf16_b8_hq16_hkv8_t4096_d128"
    w = synth.WORKLOADS[name]
    say(f"full-size {name}")
    x = synth.make_workload(w, DEV)
    out = plx.prefill(x["q"], x["k"], x["v"], x["rho"])
    torch.cuda.synchronize()
    h = {n: host64(x[n]) for n in ("q", "k", "v", "rho")}
    tau = 1 / np.sqrt(w.d)
    t0 = time.time()
    ref = oracle.prefill(h["q"], h["k"], h["v"], h["rho"], tau)
    say(f"  oracle: all {w.B * w.Hq * w.T} rows in {time.time() - t0:.1f} s on {oracle.num_threads()} threads")
    got = host64(out)
    assert_close(got, ref, w.dtype, f"{name}: all {w.B * w.Hq * w.T} rows")
    # the explicit form on 64+ rows: first and last positions, block edges, random
    rng = np.random.default_rng(6)
    ts = sorted({0, 1, 63, 64, 2047, 2048, w.T - 2, w.T - 1} | set(int(t) for t in rng.integers(0, w.T, 4)))
    rows = np.array([(b, hh, t) for b in (0, w.B - 1) for hh in (0, 5, 10, w.Hq - 1) for t in ts], dtype=np.int64)
    exp = oracle.prefill(h["q"], h["k"], h["v"], h["rho"], tau, form=oracle.EXPLICIT, rows=rows)
    _forms_agree(ref[rows[:, 0], rows[:, 1], rows[:, 2]], exp, name)
    assert_close(got[rows[:, 0], rows[:, 1], rows[:, 2]], exp, w.dtype, f"{name}: {len(rows)} rows vs explicit")
    del h, ref, got

    # rho = 0 at full size: bitwise the softmax-only kernel
    say("  rho = 0 vs softmax-only at full size")
    zero = torch.zeros_like(x["rho"])
    a = plx.prefill(x["q"], x["k"], x["v"], zero)
    b = plx.prefill(x["q"], x["k"], x["v"], None)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_prefill_f32_every_row_both_forms():
    """The fp32 workload: every row against both oracle forms (max-abs 1e-5)."""
    name = "prefill_f32_b1_h2_t256_d64"
    w = synth.WORKLOADS[name]
    say(f"full-size {name}")
    x = synth.make_workload(w, DEV)
    out = plx.prefill(x["q"], x["k"], x["v"], x["rho"])
    torch.cuda.synchronize()
    h = {n: host64(x[n]) for n in ("q", "k", "v", "rho")}
    tau = 1 / np.sqrt(w.d)
    ref = oracle.prefill(h["q"], h["k"], h["v"], h["rho"], tau)
    exp = oracle.prefill(h["q"], h["k"], h["v"], h["rho"], tau, form=oracle.EXPLICIT)
    _forms_agree(ref.reshape(-1, w.d), exp.reshape(-1, w.d), name)
    for r, what in ((ref, "expanded"), (exp, "explicit")):
        assert_close(host64(out), r, w.dtype, f"{name}: all {w.Hq * w.T} rows vs {what} form")


def test_prefill_beyond_2_31_elements():
    """q, rho and out of 72 x 16 x 16384 x 128 = 2.4e9 elements each: the last
    sequence's rows start at element 71 * 2^25 > 2^31, so every offset must
    be 64-bit.  Sampled rows of the first and last sequences and of three
    heads, at the first, last and block-edge positions, against the oracle."""
    B, Hq, Hkv, T, d = 72, 16, 8, 16384, 128
    say(f"prefill past 2^31 elements: B={B} Hq={Hq} Hkv={Hkv} T={T} d={d} ({B * Hq * T * d} elements per q)")
    x = synth.make_prefill(B, Hq, Hkv, T, d, torch.bfloat16, DEV, seed=21)
    out = plx.prefill(x["q"], x["k"], x["v"], x["rho"])
    torch.cuda.synchronize()
    bs = [0, B - 1]
    heads = [0, 5, Hq - 1]
    ts = [0, 1, 63, 64, 4095, 8191, 8192, T - 65, T - 1]
    sub = {n: x[n][bs] for n in ("q", "k", "v", "rho")}
    rows = np.array([(i, h, t) for i in range(len(bs)) for h in heads for t in ts], dtype=np.int64)
    ref = oracle.prefill(host64(sub["q"]), host64(sub["k"]), host64(sub["v"]), host64(sub["rho"]), 1 / np.sqrt(d),
                         rows=rows)
    got = host64(out[bs])[rows[:, 0], rows[:, 1], rows[:, 2]]
    del x, out, sub
    assert_close(got, ref, torch.bfloat16, f"prefill past 2^31: {len(rows)} rows")
