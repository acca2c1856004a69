"""libparallax driven from plain C: tests/c/abi_check.c (built by the build
step with gcc against libparallax.so and the HIP runtime's C API) reads seeded
inputs from raw bf16 files, calls parallax_fwd_decode (contiguous and ragged)
and parallax_fwd_prefill, checks that rejected calls return their status
codes, and writes the output; this test compares it with the fp64 oracle.
No Python binding is involved in the calls."""
import os
import subprocess
import tempfile

import numpy as np
import pytest
import torch

import oracle
from transformer_attention_flash_amd import synth

from gpu_common import assert_close, gpu_available, host64, say

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

BIN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c", "abi_check")
BF = torch.bfloat16


def _write(dirn, name, t):
    t.contiguous().cpu().view(torch.int16).numpy().tofile(os.path.join(dirn, name))


def _run(mode, dirn, shape, *dims):
    if not os.path.exists(BIN):
        pytest.fail(f"{BIN} is not built (the build step compiles it)")
    res = subprocess.run([BIN, mode, dirn, *map(str, dims)], capture_output=True, text=True, timeout=120)
    say(res.stdout.strip(), res.stderr.strip())
    assert res.returncode == 0, f"abi_check {mode} failed: {res.stderr}"
    raw = np.fromfile(os.path.join(dirn, "out.bin"), dtype=np.int16)
    return host64(torch.from_numpy(raw).view(BF).reshape(shape))


def test_decode_contiguous_from_c():
    B, Hq, Hkv, L, d = 3, 8, 4, 700, 128
    say(f"C ABI: decode B={B} Hq={Hq} Hkv={Hkv} L={L} d={d}")
    x = synth.make_decode(B, Hq, Hkv, L, d, BF, "cpu", seed=11)
    with tempfile.TemporaryDirectory() as dirn:
        for n in ("q", "k", "v", "rho"):
            _write(dirn, f"{n}.bin", x[n])
        got = _run("decode", dirn, (B, Hq, d), B, Hq, Hkv, L, d)
    ref = oracle.decode(host64(x["q"]), host64(x["rho"]), host64(x["k"]), host64(x["v"]), 1 / np.sqrt(d))
    assert_close(got, ref, BF, "decode from C")


def test_decode_ragged_from_c():
    lengths = [0, 5, 300, 1000]
    Hq, Hkv, d = 4, 2, 64
    say(f"C ABI: ragged decode lengths={lengths} Hq={Hq} Hkv={Hkv} d={d}")
    x = synth.make_decode_ragged(torch.tensor(lengths, dtype=torch.int64), Hq, Hkv, d, BF, "cpu", seed=12)
    with tempfile.TemporaryDirectory() as dirn:
        for n in ("q", "k", "v", "rho"):
            _write(dirn, f"{n}.bin", x[n])
        x["cu_host"].numpy().astype(np.int64).tofile(os.path.join(dirn, "cu.bin"))
        got = _run("ragged", dirn, (len(lengths), Hq, d), len(lengths), Hq, Hkv, x["max_ctx"], d)
    ref = oracle.decode(host64(x["q"]), host64(x["rho"]), host64(x["k"]), host64(x["v"]), 1 / np.sqrt(d),
                        cu_seqlens=x["cu_host"].numpy(), Hkv=Hkv)
    assert_close(got, ref, BF, "ragged decode from C")
    assert (got[0] == 0).all(), "the empty sequence must give zeros"


def test_prefill_from_c():
    B, Hq, Hkv, T, d = 1, 4, 2, 200, 128
    say(f"C ABI: prefill B={B} Hq={Hq} Hkv={Hkv} T={T} d={d}")
    x = synth.make_prefill(B, Hq, Hkv, T, d, BF, "cpu", seed=13)
    with tempfile.TemporaryDirectory() as dirn:
        for n in ("q", "k", "v", "rho"):
            _write(dirn, f"{n}.bin", x[n])
        got = _run("prefill", dirn, (B, Hq, T, d), B, Hq, Hkv, T, d)
    ref = oracle.prefill(host64(x["q"]), host64(x["k"]), host64(x["v"]), host64(x["rho"]), 1 / np.sqrt(d))
    assert_close(got, ref, BF, "prefill from C")
