"""GPU parity: libparallax (through the C ABI) against the fp64 oracle.

Small cases span several key tiles, several query blocks and chunks, ragged
tails, every supported group size and head dimension, and the degenerate
cases (one key, empty sequences).  Each compares every output element.
"""
import numpy as np
import pytest
import torch

import oracle
import transformer_attention_flash_amd as plx
from transformer_attention_flash_amd import synth

from gpu_common import assert_close, assert_within_bound, bound_decode, bound_prefill, host64, say

pytestmark = pytest.mark.gpu

DEV = "cuda"
BF, F32 = torch.bfloat16, torch.float32


@pytest.fixture(scope="module", autouse=True)
def _require_gpu():
    if not torch.cuda.is_available():
        pytest.fail("these tests need a GPU (they run the HIP library)")
    plx.load_library()


def _tau(d):
    return 1.0 / np.sqrt(d)


# ---------------------------------------------------------------------------
# decode, contiguous cache
# ---------------------------------------------------------------------------

DECODE_CASES = [
    # B, Hq, Hkv, L, d, dtype, keys_per_split
    (2, 4, 2, 300, 128, BF, 0),
    (2, 4, 2, 300, 128, BF, 64),     # 5 chunks, ragged last chunk
    (3, 2, 2, 77, 64, BF, 32),       # G = 1
    (2, 16, 2, 129, 64, BF, 0),      # G = 8
    (2, 16, 4, 200, 128, BF, 96),    # G = 4
    (1, 2, 1, 1, 128, BF, 0),        # a single key
    (1, 8, 2, 1000, 64, BF, 0),
    (2, 4, 2, 300, 128, F32, 64),
    (2, 4, 4, 64, 64, F32, 0),
    (1, 8, 1, 45, 128, F32, 32),     # G = 8, fp32
    (2, 4, 2, 4096, 128, BF, 32),    # 128 chunks per sequence: the merge's wavefronts each sum 32
    (1, 4, 2, 32768, 64, BF, 32),    # 1024 chunks per sequence
]


@pytest.mark.parametrize("case", DECODE_CASES, ids=[str(c[:6]) + f"-ks{c[6]}" for c in DECODE_CASES])
def test_decode_contiguous(case):
    B, Hq, Hkv, L, d, dtype, ks = case
    say(f"decode contiguous {case}")
    x = synth.make_decode(B, Hq, Hkv, L, d, dtype, DEV, seed=1)
    out = plx.decode(x["q"], x["k"], x["v"], x["rho"], keys_per_split=ks)
    torch.cuda.synchronize()
    ref = oracle.decode(host64(x["q"]), host64(x["rho"]), host64(x["k"]), host64(x["v"]), _tau(d))
    assert_close(host64(out), ref, dtype, f"decode {case}")
    if L == 1:  # one key: o = v_0 whatever q and rho are
        G = Hq // Hkv
        v0 = host64(x["v"])[:, :, 0, :].repeat(G, axis=1)
        assert_close(host64(out), v0, dtype, "single key equals its value")


RAGGED_CASES = [
    # lengths, Hq, Hkv, d, keys_per_split, dtype
    ([0, 1, 31, 32, 33, 257, 1000], 4, 2, 64, 0, BF),
    ([0, 1, 31, 32, 33, 257, 1000], 4, 2, 128, 64, BF),
    ([700, 5, 0, 0, 129], 8, 4, 128, 32, BF),
    ([64, 3000, 17], 16, 2, 64, 0, BF),
    ([0, 3, 200, 777], 8, 2, 128, 0, F32),
    ([1, 129, 64], 4, 4, 64, 32, F32),
    # chunks of 512 and 1024 keys run 4-wavefront workgroups; sequences shorter
    # than 97 keys leave some of their wavefronts without keys for the merge
    ([0, 1, 5, 40, 70, 97, 600, 1500], 8, 4, 128, 512, BF),
    ([3, 64, 2100], 4, 2, 64, 1024, BF),
]


@pytest.mark.parametrize("case", RAGGED_CASES, ids=[f"r{i}" for i in range(len(RAGGED_CASES))])
def test_decode_ragged(case):
    lengths, Hq, Hkv, d, ks, dtype = case
    say(f"decode ragged {case}")
    lens = torch.tensor(lengths, dtype=torch.int64)
    x = synth.make_decode_ragged(lens, Hq, Hkv, d, dtype, DEV, seed=2)
    out = plx.decode(x["q"], x["k"], x["v"], x["rho"], cu_seqlens=x["cu_seqlens"], max_ctx=x["max_ctx"],
                     num_kv_heads=Hkv, keys_per_split=ks)
    torch.cuda.synchronize()
    ref = oracle.decode(host64(x["q"]), host64(x["rho"]), host64(x["k"]), host64(x["v"]), _tau(d),
                        cu_seqlens=x["cu_host"].numpy(), Hkv=Hkv)
    got = host64(out)
    assert_close(got, ref, dtype, f"ragged {case}")
    for b, n in enumerate(lengths):
        if n == 0:
            assert (got[b] == 0).all(), "an empty sequence must give zeros"


@pytest.mark.parametrize("ragged", [False, True])
def test_decode_all_sequences_empty(ragged):
    """A batch whose caches hold no key at all (max_ctx = 0): the cache
    tensors have no storage, and every output row is zero."""
    say(f"decode, every sequence empty, ragged={ragged}")
    B, Hq, Hkv, d = 3, 4, 2, 128
    if ragged:
        x = synth.make_decode_ragged(torch.zeros(B, dtype=torch.int64), Hq, Hkv, d, BF, DEV, seed=4)
        x["k"] = torch.empty(0, dtype=BF, device=DEV)
        x["v"] = torch.empty(0, dtype=BF, device=DEV)
        kw = dict(cu_seqlens=x["cu_seqlens"], max_ctx=0, num_kv_heads=Hkv)
    else:
        x = synth.make_decode(B, Hq, Hkv, 0, d, BF, DEV, seed=4)
        kw = {}
    assert x["k"].numel() == 0
    for rho in (x["rho"], None):
        out = torch.full_like(x["q"], 7.0)
        plx.decode(x["q"], x["k"], x["v"], rho, out=out, **kw)
        torch.cuda.synchronize()
        assert torch.count_nonzero(out).item() == 0


def test_decode_rho_none_is_bitwise_zero_probe():
    say("decode rho=None vs rho=0")
    x = synth.make_decode(4, 16, 8, 1000, 128, BF, DEV, seed=3)
    for ks in (0, 64):
        a = plx.decode(x["q"], x["k"], x["v"], None, keys_per_split=ks)
        b = plx.decode(x["q"], x["k"], x["v"], torch.zeros_like(x["rho"]), keys_per_split=ks)
        torch.cuda.synchronize()
        assert torch.equal(a, b), f"keys_per_split={ks}"
    # reference attention on the CPU in fp32
    ref = torch.nn.functional.scaled_dot_product_attention(
        x["q"].cpu().float()[:, :, None, :], x["k"].cpu().float(), x["v"].cpu().float(),
        enable_gqa=True)[:, :, 0, :]
    assert_close(host64(a), host64(ref), BF, "rho=None vs torch fp32 softmax attention")


def test_decode_chunking_is_consistent():
    """Every chunk size gives the oracle's answer; repeated calls are bitwise equal."""
    say("decode chunk sweep")
    x = synth.make_decode(2, 8, 4, 2000, 128, BF, DEV, seed=4)
    ref = oracle.decode(host64(x["q"]), host64(x["rho"]), host64(x["k"]), host64(x["v"]), _tau(128))
    for ks in (32, 96, 256, 2048, 4096):
        a = plx.decode(x["q"], x["k"], x["v"], x["rho"], keys_per_split=ks)
        b = plx.decode(x["q"], x["k"], x["v"], x["rho"], keys_per_split=ks)
        torch.cuda.synchronize()
        assert torch.equal(a, b), f"non-deterministic at keys_per_split={ks}"
        assert_close(host64(a), ref, BF, f"ks={ks}")


# ---------------------------------------------------------------------------
# causal prefill
# ---------------------------------------------------------------------------

PREFILL_CASES = [
    # B, Hq, Hkv, T, d, dtype
    (1, 2, 2, 256, 64, F32),         # the fp32 workload at its full size
    (2, 4, 2, 200, 128, BF),
    (1, 2, 2, 333, 64, BF),          # G = 1
    (1, 8, 2, 130, 128, BF),         # G = 4
    (1, 16, 2, 70, 64, BF),          # G = 8
    (1, 4, 2, 100, 128, F32),
    (2, 2, 1, 1, 64, BF),            # T = 1
    (1, 2, 1, 513, 128, BF),
    (1, 8, 2, 150, 128, F32),        # fp32, G = 4
    (1, 16, 2, 77, 64, F32),         # fp32, G = 8
    (2, 8, 8, 3, 64, F32),           # fp32, T < one key tile
]


@pytest.mark.parametrize("case", PREFILL_CASES, ids=[str(c) for c in PREFILL_CASES])
def test_prefill(case):
    B, Hq, Hkv, T, d, dtype = case
    say(f"prefill {case}")
    gen_dev = "cpu" if dtype == F32 else DEV  # the fp32 workload is drawn on the CPU
    x = synth.make_prefill(B, Hq, Hkv, T, d, dtype, gen_dev, seed=0)
    x = {k: v.to(DEV) for k, v in x.items()}
    out = plx.prefill(x["q"], x["k"], x["v"], x["rho"])
    torch.cuda.synchronize()
    ref = oracle.prefill(host64(x["q"]), host64(x["k"]), host64(x["v"]), host64(x["rho"]), _tau(d))
    got = host64(out)
    assert_close(got, ref, dtype, f"prefill {case}")
    G = Hq // Hkv
    v0 = host64(x["v"])[:, :, 0, :].repeat(G, axis=1)
    assert_close(got[:, :, 0, :], v0, dtype, "row t=0 equals v_0")


@pytest.mark.parametrize("dtype", [BF, F32])
def test_prefill_rho_zero_is_bitwise_softmax_only(dtype):
    say(f"prefill rho=0 vs softmax-only {dtype}")
    x = synth.make_prefill(2, 8, 4, 300, 128, dtype, DEV, seed=5)
    a = plx.prefill(x["q"], x["k"], x["v"], None)
    b = plx.prefill(x["q"], x["k"], x["v"], torch.zeros_like(x["rho"]))
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    ref = torch.nn.functional.scaled_dot_product_attention(
        x["q"].cpu().float(), x["k"].cpu().float(), x["v"].cpu().float(), is_causal=True, enable_gqa=True)
    assert_close(host64(a), host64(ref), dtype, "softmax-only vs torch fp32 causal attention")


@pytest.mark.parametrize("dtype", [BF, F32])
def test_prefill_sharp_scores(dtype):
    """Queries scaled by 8 (exact in both dtypes): scores ~ N(0, 64), so along a
    row the running max rises past the rescale slack many times and the
    weights span many orders of magnitude; one late key per KV head is also
    aligned with the query rows to force a rescale well inside the row."""
    d = 128 if dtype == BF else 64
    say(f"prefill sharp scores {dtype}")
    gen_dev = "cpu" if dtype == F32 else DEV
    x = synth.make_prefill(1, 4, 2, 600, d, dtype, gen_dev, seed=8)
    x = {k: v.to(DEV) for k, v in x.items()}
    x["q"] = x["q"] * 8
    x["k"][:, :, 450, :] = x["q"][:, 0::2, 450, :] / 8  # key 450 of KV head g aligned with query head 2g
    out = plx.prefill(x["q"], x["k"], x["v"], x["rho"])
    torch.cuda.synchronize()
    h = {n: host64(x[n]) for n in ("q", "k", "v", "rho")}
    ref = oracle.prefill(h["q"], h["k"], h["v"], h["rho"], _tau(d))
    bound = bound_prefill(h["q"], h["k"], h["v"], h["rho"], _tau(d), dtype)
    assert_within_bound(host64(out), ref, bound, f"prefill sharp {dtype}")


def test_decode_sharp_scores():
    """Decode with scores ~ N(0, 64) and one late aligned key, split into chunks
    whose maxima differ by large amounts (the merge rescales them)."""
    say("decode sharp scores")
    x = synth.make_decode(2, 8, 4, 3000, 128, BF, DEV, seed=9)
    x["q"] = x["q"] * 8
    x["k"][:, :, 2900, :] = x["q"][:, 0::2, :] / 8
    h = {n: host64(x[n]) for n in ("q", "k", "v", "rho")}
    ref = oracle.decode(h["q"], h["rho"], h["k"], h["v"], _tau(128))
    for ks in (0, 256):
        out = plx.decode(x["q"], x["k"], x["v"], x["rho"], keys_per_split=ks)
        torch.cuda.synchronize()
        bound = bound_decode(h["q"], h["rho"], h["k"], h["v"], _tau(128), BF, n_merge=1 if ks == 0 else 2)
        assert_within_bound(host64(out), ref, bound, f"decode sharp ks={ks}")


# More items than CUs: the bf16 kernel with a probe then runs its persistent
# loop (one workgroup per CU, items paired long/short per XCD, the next item's
# q and rho requested during the last tile).  Ragged T for every group size;
# with G = 1 the first wavefronts of a workgroup have no rows in its last tile.
PERSISTENT_CASES = [
    # B, Hq, Hkv, T, d: items = B * Hkv * ceil(T / (128 / G))
    (2, 8, 8, 2100, 64),      # G = 1: 272 items
    (1, 16, 4, 2100, 128),    # G = 4: 264 items
    (1, 16, 2, 2100, 128),    # G = 8: 264 items
    (3, 16, 8, 1500, 128),    # G = 2: 576 items
]


@pytest.mark.parametrize("case", PERSISTENT_CASES, ids=[str(c) for c in PERSISTENT_CASES])
def test_prefill_persistent_grid_ragged(case):
    B, Hq, Hkv, T, d = case
    say(f"prefill persistent grid {case}")
    x = synth.make_prefill(B, Hq, Hkv, T, d, BF, DEV, seed=11)
    out = plx.prefill(x["q"], x["k"], x["v"], x["rho"])
    zero = plx.prefill(x["q"], x["k"], x["v"], torch.zeros_like(x["rho"]))
    soft = plx.prefill(x["q"], x["k"], x["v"], None)
    torch.cuda.synchronize()
    ref = oracle.prefill(host64(x["q"]), host64(x["k"]), host64(x["v"]), host64(x["rho"]), _tau(d))
    assert_close(host64(out), ref, BF, f"prefill persistent {case}")
    # the persistent probe kernel with rho = 0 against the one-item softmax-only kernel
    assert torch.equal(zero, soft)


def test_prefill_deterministic():
    say("prefill determinism")
    x = synth.make_prefill(1, 16, 8, 700, 128, BF, DEV, seed=6)
    a = plx.prefill(x["q"], x["k"], x["v"], x["rho"])
    b = plx.prefill(x["q"], x["k"], x["v"], x["rho"])
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_stream_argument_is_honoured():
    say("explicit stream")
    x = synth.make_decode(2, 4, 2, 500, 64, BF, DEV, seed=7)
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        a = plx.decode(x["q"], x["k"], x["v"], x["rho"])
    s.synchronize()
    b = plx.decode(x["q"], x["k"], x["v"], x["rho"])
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_concurrent_calls_on_two_streams():
    """The library keeps no state between calls: decodes (each with its own
    workspace, several chunks so the merge kernel runs) and prefills issued
    on two streams at once give the same bits as the same calls run one
    after another."""
    say("two streams at once")
    xd = [synth.make_decode(3, 8, 4, 1500, 128, BF, DEV, seed=20 + i) for i in range(2)]
    xp = [synth.make_prefill(1, 4, 2, 300, 128, BF, DEV, seed=30 + i) for i in range(2)]
    ref_d = [plx.decode(x["q"], x["k"], x["v"], x["rho"], keys_per_split=256) for x in xd]
    ref_p = [plx.prefill(x["q"], x["k"], x["v"], x["rho"]) for x in xp]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    got_d, got_p = [None, None], [None, None]
    for rep in range(3):
        for i, s in enumerate(streams):
            with torch.cuda.stream(s):
                got_d[i] = plx.decode(xd[i]["q"], xd[i]["k"], xd[i]["v"], xd[i]["rho"], keys_per_split=256)
                got_p[i] = plx.prefill(xp[i]["q"], xp[i]["k"], xp[i]["v"], xp[i]["rho"])
        torch.cuda.synchronize()
        for i in range(2):
            assert torch.equal(got_d[i], ref_d[i]), f"decode on stream {i}, repetition {rep}"
            assert torch.equal(got_p[i], ref_p[i]), f"prefill on stream {i}, repetition {rep}"
