"""fp64 CPU oracle of the Parallax attention forward pass.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the CPU-baseline leg
of the benchmark may import this package; the product library never does.  It
shares no code with the HIP path.

The arithmetic lives in ``parallax_oracle.c`` (plain C, fp64, OpenMP over rows).
This module compiles it (``gcc``), loads it with ctypes and maps the two call
shapes of the method onto independent query rows:

* causal prefill: row (b, h, t) attends keys 0..t of KV head h // G
  (G = Hq / Hkv), the diagonal included;
* decode: row (b, h) attends all L_b cached keys of KV head h // G, from a
  contiguous cache [B, Hkv, L, d] or from packed per-sequence slabs
  [Hkv, L_b, d] whose token offsets are ``cu_seqlens``.

Method: the gist.science technical summary of Parallax ("Method: Parallax /
core mechanism") gives o_i = o^SA_i - Sigma^(i)_KV rho_i; the news.chathome.org
article ("How does the mechanism work?") and the same summary ("key design
choices") set the boundary-amplification factor to zero.  Causal masking and
the GQA head mapping are readings (the pages are silent): the language-model
setting of the news.chathome.org article ("Experiments") implies a causal
decoder, and query head h shares KV head h // G as in grouped-query attention.

Every input is upcast exactly to float64 before it reaches the C code.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "parallax_oracle.c")
_LIB = os.path.join(_HERE, "libparallax_oracle.so")

EXPLICIT = 0
EXPANDED = 1

_lib = None


def build(force: bool = True) -> str:
    """Compile the C oracle into oracle/libparallax_oracle.so (gcc, -O2, OpenMP,
    IEEE fp64: no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        cmd = ["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared",
               "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _bind(lib):
    dp = ctypes.POINTER(ctypes.c_double)
    ip = ctypes.POINTER(ctypes.c_int64)
    lib.plx_oracle_rows.argtypes = [dp, dp, dp, dp, ip, ip, ctypes.c_int64,
                                    ctypes.c_int64, ctypes.c_int32, ctypes.c_double,
                                    ctypes.c_int32, dp]
    lib.plx_oracle_rows.restype = ctypes.c_int
    lib.plx_oracle_num_threads.restype = ctypes.c_int
    lib.plx_oracle_set_num_threads.argtypes = [ctypes.c_int]
    return lib


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        _lib = _bind(ctypes.CDLL(_LIB))
    return _lib


def load_variant(path: str):
    """Load another build of the same C source (the tests use this to check
    that deliberately broken copies of the oracle fail the pins)."""
    return _bind(ctypes.CDLL(path))


def num_threads() -> int:
    return int(_load().plx_oracle_num_threads())


def set_num_threads(n: int) -> None:
    _load().plx_oracle_set_num_threads(int(n))


def _f64(a):
    a = np.asarray(a)
    if a.dtype != np.float64:
        a = a.astype(np.float64)  # exact for bf16/fp16/fp32 inputs
    return np.ascontiguousarray(a)


def _ptr(a):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def attend_rows(q_rows, rho_rows, k_base, v_base, key_off, key_len, key_stride,
                tau: float, form: int = EXPANDED, lib=None):
    """Evaluate independent query rows.

    q_rows, rho_rows: [n, d] (rho_rows may be None: a zero probe).
    k_base, v_base:   flat key/value storage; row i uses key_len[i] keys that
                      start at element key_off[i], key_stride elements apart.
    Returns out [n, d] float64.
    """
    q_rows = _f64(q_rows)
    n, d = q_rows.shape
    rho_rows = None if rho_rows is None else _f64(rho_rows)
    if rho_rows is not None and rho_rows.shape != (n, d):
        raise ValueError("rho_rows must match q_rows")
    k_base = _f64(k_base).reshape(-1)
    v_base = _f64(v_base).reshape(-1)
    if k_base.size != v_base.size:
        raise ValueError("k and v storage differ in size")
    key_off = np.ascontiguousarray(np.asarray(key_off, dtype=np.int64).reshape(-1))
    key_len = np.ascontiguousarray(np.asarray(key_len, dtype=np.int64).reshape(-1))
    if key_off.size != n or key_len.size != n:
        raise ValueError("key_off/key_len must have one entry per row")
    if n:
        if (key_off < 0).any() or (key_len < 0).any():
            raise ValueError("negative key offset or length")
        used = key_len > 0  # an empty row reads no key
        last = key_off[used] + (key_len[used] - 1) * key_stride + d
        if last.size and int(last.max()) > k_base.size:
            raise ValueError("a row's keys fall outside the key storage")
    out = np.zeros((n, d), dtype=np.float64)
    if n == 0:
        return out
    rc = (lib or _load()).plx_oracle_rows(
        _ptr(q_rows), None if rho_rows is None else _ptr(rho_rows), _ptr(k_base), _ptr(v_base),
        key_off.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
        key_len.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
        int(key_stride), int(n), int(d), float(tau), int(form), _ptr(out))
    if rc != 0:
        raise RuntimeError(f"plx_oracle_rows failed with code {rc}")
    return out


def prefill(q, k, v, rho, tau: float, form: int = EXPANDED, rows=None, lib=None):
    """Causal prefill.  q, rho: [B, Hq, T, d]; k, v: [B, Hkv, T, d].

    rows: optional integer array [n, 3] of (b, h, t) to evaluate; returns
    [n, d].  Without it every row is evaluated and [B, Hq, T, d] returned.
    """
    q = np.asarray(q)
    B, Hq, T, d = q.shape
    Hkv = np.asarray(k).shape[1]
    if np.asarray(k).shape != (B, Hkv, T, d) or np.asarray(v).shape != (B, Hkv, T, d):
        raise ValueError("k and v must be [B, Hkv, T, d]")
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    G = Hq // Hkv
    if rows is None:
        b, h, t = np.meshgrid(np.arange(B), np.arange(Hq), np.arange(T), indexing="ij")
        sel = np.stack([b.ravel(), h.ravel(), t.ravel()], axis=1)
    else:
        sel = np.asarray(rows, dtype=np.int64).reshape(-1, 3)
    b, h, t = sel[:, 0], sel[:, 1], sel[:, 2]
    q_rows = _f64(q)[b, h, t]
    rho_rows = None if rho is None else _f64(rho)[b, h, t]
    key_off = ((b * Hkv + h // G) * T) * d
    key_len = t + 1
    out = attend_rows(q_rows, rho_rows, k, v, key_off, key_len, d, tau, form, lib=lib)
    return out.reshape(B, Hq, T, d) if rows is None else out


def decode(q, rho, k, v, tau: float, cu_seqlens=None, Hkv=None, form: int = EXPANDED,
           rows=None, lib=None):
    """Decode: one query row per (b, h) over a KV cache.

    q, rho: [B, Hq, d].  Contiguous cache (cu_seqlens None): k, v [B, Hkv, L, d].
    Ragged cache (Hkv required): k, v are flat packed slabs, slab b =
    [Hkv, L_b, d] starting at element cu_seqlens[b] * Hkv * d, with
    L_b = cu_seqlens[b+1] - cu_seqlens[b].
    rows: optional [n, 2] of (b, h); returns [n, d], else [B, Hq, d].
    """
    q = np.asarray(q)
    B, Hq, d = q.shape
    if cu_seqlens is None:
        kk = np.asarray(k)
        if kk.ndim != 4 or kk.shape[0] != B or kk.shape[3] != d:
            raise ValueError("contiguous k must be [B, Hkv, L, d]")
        Hkv, L = kk.shape[1], kk.shape[2]
        starts = np.arange(B, dtype=np.int64) * L
        lens = np.full(B, L, dtype=np.int64)
    else:
        cu = np.asarray(cu_seqlens, dtype=np.int64)
        if cu.shape != (B + 1,):
            raise ValueError("cu_seqlens must have B + 1 entries")
        if Hkv is None:
            raise ValueError("a ragged cache needs Hkv")
        starts = cu[:-1]
        lens = cu[1:] - cu[:-1]
        if (lens < 0).any() or cu[0] != 0:
            raise ValueError("cu_seqlens must start at 0 and not decrease")
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    G = Hq // Hkv
    if rows is None:
        b, h = np.meshgrid(np.arange(B), np.arange(Hq), indexing="ij")
        sel = np.stack([b.ravel(), h.ravel()], axis=1)
    else:
        sel = np.asarray(rows, dtype=np.int64).reshape(-1, 2)
    b, h = sel[:, 0], sel[:, 1]
    q_rows = _f64(q)[b, h]
    rho_rows = None if rho is None else _f64(rho)[b, h]
    key_off = (starts[b] * Hkv + (h // G) * lens[b]) * d
    key_len = lens[b]
    out = attend_rows(q_rows, rho_rows, k, v, key_off, key_len, d, tau, form, lib=lib)
    return out.reshape(B, Hq, d) if rows is None else out
