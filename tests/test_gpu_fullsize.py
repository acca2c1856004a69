"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times (library-chosen chunking), against the fp64 oracle on sampled
rows: the oracle evaluates whole sampled sequences, read back from the device,
so its GQA / causal / ragged mapping is its own.  Sampled rows always include
the first and last sequence, and for prefill the first and last positions and
query-block edges; for the ragged batch the shortest and longest sequences.
"""
import numpy as np
import pytest
import torch

import oracle
import transformer_attention_flash_amd as plx
from transformer_attention_flash_amd import synth

from gpu_common import assert_close, host64, say

pytestmark = pytest.mark.gpu
DEV = "cuda"


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


@pytest.mark.parametrize("name,nseq", [("decode_bf16_b64_hq16_hkv8_l4096_d128", 8),
                                       ("decode_bf16_b2048_hq16_hkv8_l128_d128", 64),
                                       ("decode_bf16_b256_hq16_hkv8_l32768_d128", 4)])
def test_decode_full_size(name, nseq):
    w = synth.WORKLOADS[name]
    say(f"full-size {name}")
    x = synth.make_workload(w, DEV)
    out = plx.decode(x["q"], x["k"], x["v"], x["rho"])
    out2 = plx.decode(x["q"], x["k"], x["v"], x["rho"])
    torch.cuda.synchronize()
    assert torch.equal(out, out2), "repeated call differs"
    assert torch.isfinite(out.float()).all()
    rng = np.random.default_rng(0)
    bs = _pick(w.B, nseq, rng, must=(0, w.B - 1))
    got = host64(out[bs])
    ref = oracle.decode(host64(x["q"][bs]), host64(x["rho"][bs]), host64(x["k"][bs]), host64(x["v"][bs]),
                        1 / np.sqrt(w.d))
    assert_close(got, ref, w.dtype, f"{name}: {len(bs)} sequences x {w.Hq} heads")


def test_ragged_decode_full_size():
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
    assert torch.isfinite(out.float()).all()
    rng = np.random.default_rng(1)
    bs = _pick(w.B, 8, rng, must=(0, w.B - 1, int(lens.argmin()), int(lens.argmax())))
    # the sampled sequences' slabs, packed again in the same layout
    per_tok = w.Hkv * w.d
    ks = [host64(x["k"][cu[b] * per_tok:cu[b + 1] * per_tok]) for b in bs]
    vs = [host64(x["v"][cu[b] * per_tok:cu[b + 1] * per_tok]) for b in bs]
    sub_cu = np.concatenate([[0], np.cumsum(lens[bs])])
    ref = oracle.decode(host64(x["q"][bs]), host64(x["rho"][bs]), np.concatenate(ks), np.concatenate(vs),
                        1 / np.sqrt(w.d), cu_seqlens=sub_cu, Hkv=w.Hkv)
    assert_close(host64(out[bs]), ref, w.dtype,
                 f"{name}: sequences {bs} (lengths {lens[bs].tolist()}) x {w.Hq} heads")


def test_prefill_full_size():
    name = "prefill_bf16_b8_hq16_hkv8_t4096_d128"
    w = synth.WORKLOADS[name]
    say(f"full-size {name}")
    x = synth.make_workload(w, DEV)
    out = plx.prefill(x["q"], x["k"], x["v"], x["rho"])
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all()
    rng = np.random.default_rng(2)
    bs = _pick(w.B, 2, rng, must=(0, w.B - 1))
    edges = [0, 1, 31, 32, 63, 64, 65, 127, 128, 1000, 2047, 2048, 4031, 4032, w.T - 2, w.T - 1]
    ts = sorted(set(edges) | set(int(t) for t in rng.integers(0, w.T, 16)))
    rows = np.array([(i, h, t) for i in range(len(bs)) for h in range(w.Hq) for t in ts], dtype=np.int64)
    ref = oracle.prefill(host64(x["q"][bs]), host64(x["k"][bs]), host64(x["v"][bs]), host64(x["rho"][bs]),
                         1 / np.sqrt(w.d), rows=rows)
    got = host64(out[bs])[rows[:, 0], rows[:, 1], rows[:, 2]]
    assert_close(got, ref, w.dtype, f"{name}: {len(rows)} rows")

    # rho = 0 at full size: bitwise the softmax-only kernel
    say("  rho = 0 vs softmax-only at full size")
    zero = torch.zeros_like(x["rho"])
    a = plx.prefill(x["q"], x["k"], x["v"], zero)
    b = plx.prefill(x["q"], x["k"], x["v"], None)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


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
