"""C-ABI checks that need no GPU: the library loads, exports every function
the headers in include/ declare, and every rejected call returns its status code
from the host-side checks (which run before any HIP call)."""
import ctypes
import glob
import os
import re

import pytest

from transformer_attention_flash_amd import _native as N

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = sorted(glob.glob(os.path.join(ROOT, "include", "*.h")))

BF16, F32 = N.PLX_DTYPE_BF16, N.PLX_DTYPE_F32
INVALID, UNSUP, WS = N.PLX_ERR_INVALID_ARGUMENT, N.PLX_ERR_UNSUPPORTED, N.PLX_ERR_WORKSPACE_TOO_SMALL
SIZE_MAX = (1 << 64) - 1

# Fake, never dereferenced device addresses: every call below is rejected by
# the host checks before anything reaches the GPU.
P = [0x10000000 * (i + 1) for i in range(16)]


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(N.LIB_PATH):
        from transformer_attention_flash_amd.build import build_library
        build_library()
    return N.load()


def _declared_functions():
    names = set()
    for path in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(path).read(), flags=re.S)
        names.update(re.findall(r"\b(parallax_\w+)\s*\(", text))
    return sorted(names)


def test_header_and_exports_agree(lib):
    declared = _declared_functions()
    assert declared == sorted(N.EXPORTS)
    out = os.popen(f"nm -D --defined-only {N.LIB_PATH}").read()
    exported = sorted(set(re.findall(r"\bT (parallax_\w+)", out)))
    assert exported == declared
    for name in declared:
        assert hasattr(lib, name)


def test_every_kernel_stub_is_defined(lib):
    """Every kernel the library launches has its host-side stub defined in the
    library itself (a device-only builtin called straight from a kernel
    template once made the host pass drop stubs silently; the library then
    failed to load on the GPU)."""
    out = os.popen(f"nm --undefined-only {N.LIB_PATH}").read()
    assert "device_stub" not in out, [l for l in out.splitlines() if "device_stub" in l][:5]


def test_status_strings(lib):
    for code in range(5):
        assert N.status_string(code)
    assert N.status_string(99) == "unknown status"


def prefill(lib, q=P[0], k=P[1], v=P[2], rho=P[3], out=P[4], B=1, Hq=4, Hkv=2, T=16, d=64, scale=0.125,
            dtype=BF16):
    return lib.parallax_fwd_prefill(q, k, v, rho, out, B, Hq, Hkv, T, d, scale, dtype, None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), INVALID), (dict(k=None), INVALID), (dict(v=None), INVALID), (dict(out=None), INVALID),
    (dict(B=0), INVALID), (dict(T=0), INVALID), (dict(T=-3), INVALID), (dict(Hq=0), INVALID),
    (dict(Hkv=0), INVALID), (dict(Hq=6, Hkv=4), INVALID), (dict(d=0), INVALID),
    (dict(scale=0.0), INVALID), (dict(scale=-1.0), INVALID), (dict(scale=float("nan")), INVALID),
    (dict(scale=float("inf")), INVALID),
    (dict(d=96), UNSUP), (dict(d=256), UNSUP), (dict(Hq=6, Hkv=2), UNSUP), (dict(Hq=32, Hkv=2), UNSUP),
    (dict(dtype=7), UNSUP),
    (dict(out=P[0]), INVALID),                 # out aliases q
    (dict(out=P[1] + 64), INVALID),            # out overlaps k
    (dict(q=P[0] + 2), INVALID), (dict(rho=P[3] + 8), INVALID), (dict(out=P[4] + 4), INVALID),  # alignment
])
def test_prefill_rejections(lib, kw, code):
    assert prefill(lib, **kw) == code


def prefill_train(lib, q=P[0], k=P[1], v=P[2], rho=P[3], out=P[4], out_sa=P[5], lse=P[6], rbar=P[7], B=1, Hq=4,
                  Hkv=2, T=16, d=64, scale=0.125, dtype=BF16):
    return lib.parallax_fwd_prefill_train(q, k, v, rho, out, out_sa, lse, rbar, B, Hq, Hkv, T, d, scale, dtype, None)


@pytest.mark.parametrize("kw,code", [
    (dict(lse=None), INVALID), (dict(rbar=None), INVALID), (dict(out_sa=None), INVALID),
    (dict(rho=None), INVALID),                 # out_sa and rbar given without rho
    (dict(rho=None, out_sa=None), INVALID),    # rbar given without rho
    (dict(dtype=F32), UNSUP), (dict(d=96), UNSUP), (dict(B=0), INVALID),
    (dict(out_sa=P[4]), INVALID),              # out_sa aliases out
    (dict(lse=P[0] + 256), INVALID),           # lse overlaps q
    (dict(rbar=P[6] + 16), INVALID),           # rbar overlaps lse
    (dict(lse=P[6] + 4), INVALID),             # alignment
])
def test_prefill_train_rejections(lib, kw, code):
    assert prefill_train(lib, **kw) == code


def backward(lib, q=P[0], k=P[1], v=P[2], rho=P[3], out=P[4], out_sa=P[5], lse=P[6], rbar=P[7], dout=P[8],
             dq=P[9], dk=P[10], dv=P[11], drho=P[12], B=1, Hq=4, Hkv=2, T=16, d=64, scale=0.125, dtype=BF16,
             ws=P[13], ws_bytes=1 << 20):
    return lib.parallax_bwd_prefill(q, k, v, rho, out, out_sa, lse, rbar, dout, dq, dk, dv, drho, B, Hq, Hkv, T, d,
                                    scale, dtype, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), INVALID), (dict(dout=None), INVALID), (dict(dq=None), INVALID), (dict(dk=None), INVALID),
    (dict(lse=None), INVALID), (dict(ws=None), INVALID),
    (dict(drho=None), INVALID),                # rho given, drho missing
    (dict(rho=None), INVALID),                 # drho/out_sa/rbar given without rho
    (dict(B=0), INVALID), (dict(T=0), INVALID), (dict(scale=0.0), INVALID), (dict(Hq=6, Hkv=4), INVALID),
    (dict(dtype=F32), UNSUP), (dict(d=32), UNSUP), (dict(Hq=48, Hkv=2), UNSUP),
    (dict(Hq=8, Hkv=1, T=1 << 28, ws_bytes=1 << 40), UNSUP),  # T * G = 2^31 rows per KV group
    (dict(ws_bytes=1023), WS),                 # needs 1 * 4 * 16 * 16 = 1024 bytes
    (dict(dq=P[0]), INVALID),                  # dq aliases q
    (dict(dv=P[10] + 32), INVALID),            # dv overlaps dk
    (dict(dk=P[13]), INVALID),                 # dk overlaps the workspace
    (dict(dq=P[9] + 8), INVALID), (dict(ws=P[13] + 4), INVALID),  # alignment
])
def test_backward_rejections(lib, kw, code):
    assert backward(lib, **kw) == code


def test_backward_rejects_partial_softmax_only(lib):
    assert backward(lib, rho=None, out_sa=None, rbar=None) == INVALID      # drho without rho
    assert backward(lib, rho=None, out_sa=None, drho=None) == INVALID      # rbar without rho


def test_backward_workspace_size(lib):
    assert lib.parallax_bwd_prefill_workspace_size(8, 16, 4096) == 8 * 16 * 4096 * 16
    assert lib.parallax_bwd_prefill_workspace_size(0, 16, 4096) == SIZE_MAX
    assert lib.parallax_bwd_prefill_workspace_size(1, 1, -1) == SIZE_MAX


def decode(lib, q=P[0], rho=P[1], k=P[2], v=P[3], cu=None, max_ctx=4096, out=P[4], B=2, Hq=4, Hkv=2, d=128,
           scale=0.088, dtype=BF16, ks=None, ws=P[5], ws_bytes=1 << 30):
    """parallax_fwd_decode, or parallax_fwd_decode_chunked when ks is given."""
    if ks is None:
        return lib.parallax_fwd_decode(q, rho, k, v, cu, max_ctx, out, B, Hq, Hkv, d, scale, dtype, ws, ws_bytes,
                                       None)
    return lib.parallax_fwd_decode_chunked(q, rho, k, v, cu, max_ctx, out, B, Hq, Hkv, d, scale, dtype, ks, ws,
                                           ws_bytes, None)


DECODE_REJECTIONS = [
    (dict(q=None), INVALID), (dict(k=None), INVALID), (dict(v=None), INVALID), (dict(out=None), INVALID),
    (dict(k=None, max_ctx=1), INVALID),        # a cache without storage is only allowed when it is empty
    (dict(B=0), INVALID), (dict(max_ctx=-1), INVALID), (dict(Hq=5, Hkv=2), INVALID),
    (dict(scale=0.0), INVALID), (dict(scale=float("nan")), INVALID),
    (dict(d=32), UNSUP), (dict(Hq=48, Hkv=2), UNSUP), (dict(dtype=3), UNSUP),
    (dict(ws=None), WS), (dict(ws_bytes=100), WS),  # B=2 x 2 KV heads x 4096 keys: the library splits
    (dict(out=P[0] + 16), INVALID),            # out overlaps q
    (dict(out=P[5]), INVALID),                 # out overlaps the workspace
    (dict(k=P[2] + 2), INVALID), (dict(ws=P[5] + 8), INVALID), (dict(cu=P[6] + 4), INVALID),  # alignment
]


@pytest.mark.parametrize("kw,code", DECODE_REJECTIONS)
def test_decode_rejections(lib, kw, code):
    assert decode(lib, **kw) == code


@pytest.mark.parametrize("kw,code", DECODE_REJECTIONS + [
    (dict(ks=16), INVALID), (dict(ks=48), INVALID), (dict(ks=-32), INVALID), (dict(ks=(1 << 20) + 32), INVALID),
])
def test_decode_chunked_rejections(lib, kw, code):
    assert decode(lib, **{"ks": 256, **kw}) == code


def decode_noalloc(lib, q=P[0], rho=P[1], k=P[2], v=P[3], cu=None, max_ctx=4096, out=P[4], B=2, Hq=4, Hkv=2,
                   d=128, scale=0.088, dtype=BF16):
    return lib.parallax_fwd_decode_noalloc(q, rho, k, v, cu, max_ctx, out, B, Hq, Hkv, d, scale, dtype, None)


@pytest.mark.parametrize("kw,code", [
    (kw, code) for kw, code in DECODE_REJECTIONS if "ws" not in kw and "ws_bytes" not in kw and kw != dict(out=P[5])
] + [
    # 64 sequences x 8 KV heads of 2^22 keys: 4 chunks of 2^20 keys each, whose partials
    # (64 x 64 heads x 4 chunks x 1036 B) exceed the fixed scratch
    (dict(B=64, Hq=64, Hkv=8, max_ctx=1 << 22), WS),
])
def test_decode_noalloc_rejections(lib, kw, code):
    """Every rejection happens in the host checks, before the first HIP call
    (this machine has no GPU, so a call that got further would fail with
    PLX_ERR_HIP instead)."""
    assert decode_noalloc(lib, **kw) == code


def test_decode_noalloc_limit_matches_header(lib):
    text = open(os.path.join(ROOT, "include", "parallax.h")).read()
    assert "#define PLX_DECODE_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)" in text
    assert N.DECODE_NOALLOC_SCRATCH_BYTES == 16 << 20
    # the largest split the library's own chunking picks for caches of up to 2^20 keys fits
    f = lib.parallax_fwd_decode_workspace_size
    worst = max(f(B, 8 * Hkv, Hkv, 128, L, BF16) for B in (1, 2, 3, 5, 7, 33, 63) for Hkv in (1, 3, 8, 64)
                for L in (257, 4097, 65537, 1 << 20))
    assert 0 < worst <= N.DECODE_NOALLOC_SCRATCH_BYTES


def test_decode_workspace_size(lib):
    f = lib.parallax_fwd_decode_workspace_size
    fc = lib.parallax_fwd_decode_chunked_workspace_size
    # single chunk: no workspace
    assert f(2048, 16, 8, 128, 128, BF16) == 0
    assert fc(4, 16, 8, 128, 100, BF16, 128) == 0
    # explicit chunks: stats (3 floats, padded to 256 B) + A and B vectors
    B, Hq, d, L, ks = 3, 8, 64, 1000, 64
    n = -(-L // ks)
    slots = B * Hq * n
    stats = (slots * 3 * 4 + 255) // 256 * 256
    assert fc(B, Hq, 4, d, L, BF16, ks) == stats + slots * 2 * d * 4
    assert fc(B, Hq, 3, d, L, BF16, ks) == SIZE_MAX     # Hq % Hkv
    assert fc(B, Hq, 4, 80, L, BF16, ks) == SIZE_MAX    # head dim
    assert fc(B, Hq, 4, d, L, BF16, 40) == SIZE_MAX     # not a multiple of 32
    # the library's own choice: the chunked query with 0, and the chunk size it reports
    for shape in [(1, 16, 8, 128, 4096), (2, 4, 2, 128, 4096), (64, 16, 8, 128, 4096), (3, 8, 4, 64, 1000)]:
        assert f(*shape, BF16) == fc(*shape, BF16, 0) == fc(*shape, BF16, lib.parallax_fwd_decode_auto_split(*shape))
    assert f(3, 8, 3, 64, 1000, BF16) == SIZE_MAX


def test_decode_auto_split(lib):
    f = lib.parallax_fwd_decode_auto_split
    assert f(2048, 16, 8, 128, 128) == 256          # one chunk, no merge
    assert f(2, 16, 8, 128, 200) == 256
    assert f(64, 16, 8, 128, 4096) == 4096          # one chunk per (b, g): no merge kernel
    assert f(256, 16, 8, 128, 32768) == 32768
    assert f(2048, 32, 16, 64, 32768) == 32768
    assert f(2048, 32, 16, 64, 30000) == 32768      # rounded up to a power of two
    assert f(1, 16, 8, 128, 4096) == 256            # few sequences: more, smaller chunks
    assert f(8, 16, 8, 128, 65536) == 8192          # 64 (b, g) units x 8 chunks = 512 workgroups
    assert f(1, 8, 8, 128, 1 << 24) == 1 << 18      # 8 units x 64 chunks = 512 workgroups
    assert f(64, 8, 8, 128, 1 << 24) == 1 << 20     # chunk capped at 2^20 keys
    assert f(2, 6, 4, 128, 100) == -INVALID
    assert f(2, 4, 2, 100, 100) == -UNSUP


def test_diag_rejections(lib):
    one = ctypes.c_int32()
    assert lib.parallax_diag_device_info(0, None, ctypes.byref(one)) == INVALID
    assert lib.parallax_diag_device_info(0, ctypes.byref(one), None) == INVALID
    f = lib.parallax_diag_stream_read
    assert f(None, 1 << 20, 1, P[1], None) == INVALID
    assert f(P[0], 1 << 20, 1, None, None) == INVALID
    assert f(P[0], 0, 1, P[1], None) == INVALID           # empty
    assert f(P[0], 1000, 1, P[1], None) == INVALID        # not a multiple of 16
    assert f(P[0] + 8, 1 << 20, 1, P[1], None) == INVALID  # misaligned source
    assert f(P[0], 1 << 20, 1, P[0] + 64, None) == INVALID  # sink inside the source
    g = lib.parallax_diag_mfma_bf16
    assert g(None, 512, 100, None) == INVALID
    assert g(P[0], 0, 100, None) == INVALID
    assert g(P[0], 512, 0, None) == INVALID
    assert g(P[0], (1 << 20) + 1, 100, None) == INVALID


def test_c_caller_builds_and_rejects_bad_usage():
    """The plain-C caller (tests/c/abi_check.c) compiles against the headers and
    links to libparallax.so; bad command lines fail before any HIP call."""
    import subprocess
    import sys
    sys.path.insert(0, ROOT)
    import __graft_entry__
    exe = __graft_entry__.build_c_abi_check()
    res = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert res.returncode == 1 and "usage" in res.stderr
    res = subprocess.run([exe, "bogus", "/nonexistent", "1", "1", "1", "1", "64"], capture_output=True, text=True,
                         timeout=60)
    assert res.returncode == 1 and "mode" in res.stderr


def test_product_does_not_use_the_oracle():
    """Only tests, the smoke check and the benchmark's CPU leg may touch oracle/."""
    pkg = os.path.join(ROOT, "transformer_attention_flash_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"^\s*(import|from)\s+oracle\b|parallax_oracle|[\"']oracle[/\"']",
                                     text, flags=re.M), f
