"""Seeded synthetic inputs for the Parallax forward pass.

This module only draws random tensors and lays them out; it holds none of the
method's arithmetic.  The GPU library and the CPU oracle both consume what it
produces (the oracle reads the rounded tensors back from the device).

Recipe: one torch.Generator per workload seeded with 0 (on the device the
tensors live on; lengths of a ragged batch come from a CPU generator drawn
first).  Draw order: lengths, q, k, v, rho.  q, k, v ~ N(0, 1) and
rho ~ N(0, 0.1^2) are drawn in fp32 and rounded to the workload dtype with
round-to-nearest-even.  The softmax scale is 1/sqrt(d).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import torch

RHO_STD = 0.1
_CHUNK = 1 << 27  # elements drawn per randn call on the device


@dataclass(frozen=True)
class Workload:
    """One benchmark / parity workload."""
    name: str
    kind: str                 # "prefill" | "decode" | "decode_ragged"
    dtype: torch.dtype
    B: int
    Hq: int
    Hkv: int
    d: int
    T: int = 0                # prefill length
    L: int = 0                # contiguous decode context
    len_lo: int = 0           # ragged decode: inclusive length range
    len_hi: int = 0
    extra: dict = field(default_factory=dict)


WORKLOADS = {
    w.name: w for w in [
        Workload("prefill_f32_b1_h2_t256_d64", "prefill", torch.float32, B=1, Hq=2, Hkv=2, d=64, T=256),
        Workload("decode_bf16_b64_hq16_hkv8_l4096_d128", "decode", torch.bfloat16, B=64, Hq=16, Hkv=8, d=128,
                 L=4096),
        Workload("decode_bf16_b2048_hq16_hkv8_l128_d128", "decode", torch.bfloat16, B=2048, Hq=16, Hkv=8,
                 d=128, L=128),
        Workload("decode_bf16_b256_hq16_hkv8_l32768_d128", "decode", torch.bfloat16, B=256, Hq=16, Hkv=8,
                 d=128, L=32768),
        Workload("prefill_bf16_b8_hq16_hkv8_t4096_d128", "prefill", torch.bfloat16, B=8, Hq=16, Hkv=8, d=128,
                 T=4096),
        Workload("decode_ragged_bf16_b2048_hq32_hkv16_d64_l128to32768", "decode_ragged", torch.bfloat16,
                 B=2048, Hq=32, Hkv=16, d=64, len_lo=128, len_hi=32768),
    ]
}


def _fill_normal(t: torch.Tensor, gen: torch.Generator, std: float = 1.0) -> torch.Tensor:
    """Fill t with N(0, std^2) drawn in fp32 chunk by chunk, rounded to t's dtype."""
    flat = t.view(-1)
    n = flat.numel()
    for s in range(0, n, _CHUNK):
        m = min(_CHUNK, n - s)
        x = torch.randn(m, generator=gen, device=t.device, dtype=torch.float32)
        if std != 1.0:
            x.mul_(std)
        flat[s:s + m].copy_(x)
    return t


def _generator(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def make_prefill(B, Hq, Hkv, T, d, dtype, device, seed: int = 0, rho_std: float = RHO_STD):
    """q, rho [B, Hq, T, d]; k, v [B, Hkv, T, d]."""
    g = _generator(device, seed)
    out = {}
    for name, shape, std in (("q", (B, Hq, T, d), 1.0), ("k", (B, Hkv, T, d), 1.0),
                             ("v", (B, Hkv, T, d), 1.0), ("rho", (B, Hq, T, d), rho_std)):
        out[name] = _fill_normal(torch.empty(shape, dtype=dtype, device=device), g, std)
    return out


def make_projection(B, T, d_model, Hq, Hkv, d, dtype, device, seed: int = 0):
    """Layer input x [B, T, d_model] ~ N(0, 1) and a stacked q/k/v/probe
    weight [(2 Hq + 2 Hkv) d, d_model] ~ N(0, 1/d_model), so projected
    features have unit variance."""
    g = _generator(device, 2000 + seed)
    x = _fill_normal(torch.empty((B, T, d_model), dtype=dtype, device=device), g)
    w = _fill_normal(torch.empty(((2 * Hq + 2 * Hkv) * d, d_model), dtype=dtype, device=device), g,
                     1.0 / d_model ** 0.5)
    return x, w


def make_upstream_grad(shape, dtype, device, seed: int = 0):
    """An upstream gradient dO ~ N(0, 1) (the backward's second input), drawn
    from its own generator seeded with 1000 + seed so it does not disturb the
    forward inputs' draw order."""
    return _fill_normal(torch.empty(shape, dtype=dtype, device=device), _generator(device, 1000 + seed))


def make_decode(B, Hq, Hkv, L, d, dtype, device, seed: int = 0, rho_std: float = RHO_STD):
    """q, rho [B, Hq, d]; contiguous k, v [B, Hkv, L, d]."""
    g = _generator(device, seed)
    out = {}
    for name, shape, std in (("q", (B, Hq, d), 1.0), ("k", (B, Hkv, L, d), 1.0), ("v", (B, Hkv, L, d), 1.0),
                             ("rho", (B, Hq, d), rho_std)):
        out[name] = _fill_normal(torch.empty(shape, dtype=dtype, device=device), g, std)
    return out


def ragged_lengths(B: int, lo: int, hi: int, seed: int = 0) -> torch.Tensor:
    """B context lengths drawn uniformly from the integers lo..hi (inclusive)."""
    g = torch.Generator()
    g.manual_seed(seed)
    return torch.randint(lo, hi + 1, (B,), generator=g, dtype=torch.int64)


def cu_from_lengths(lengths: torch.Tensor) -> torch.Tensor:
    """Token offsets [B + 1] of packed sequences (int64, CPU)."""
    cu = torch.zeros(lengths.numel() + 1, dtype=torch.int64)
    cu[1:] = torch.cumsum(lengths.to(torch.int64), 0)
    return cu


def make_decode_ragged(lengths: torch.Tensor, Hq, Hkv, d, dtype, device, seed: int = 0,
                       rho_std: float = RHO_STD, gen: Optional[torch.Generator] = None):
    """Ragged cache: packed slabs [Hkv, L_b, d] back to back, cu_seqlens on the device.

    k and v are flat tensors of sum(L_b) * Hkv * d elements.
    """
    B = lengths.numel()
    cu = cu_from_lengths(lengths)
    n_tok = int(cu[-1])
    g = gen if gen is not None else _generator(device, seed)
    out = {"q": _fill_normal(torch.empty((B, Hq, d), dtype=dtype, device=device), g)}
    out["k"] = _fill_normal(torch.empty(max(n_tok * Hkv * d, 1), dtype=dtype, device=device), g)
    out["v"] = _fill_normal(torch.empty(max(n_tok * Hkv * d, 1), dtype=dtype, device=device), g)
    out["rho"] = _fill_normal(torch.empty((B, Hq, d), dtype=dtype, device=device), g, rho_std)
    out["cu_seqlens"] = cu.to(device)
    out["cu_host"] = cu
    out["max_ctx"] = int(lengths.max()) if B else 0
    return out


def make_workload(w: Workload, device, seed: int = 0):
    if w.kind == "prefill":
        return make_prefill(w.B, w.Hq, w.Hkv, w.T, w.d, w.dtype, device, seed)
    if w.kind == "decode":
        return make_decode(w.B, w.Hq, w.Hkv, w.L, w.d, w.dtype, device, seed)
    if w.kind == "decode_ragged":
        lengths = ragged_lengths(w.B, w.len_lo, w.len_hi, seed)
        return make_decode_ragged(lengths, w.Hq, w.Hkv, w.d, w.dtype, device, seed)
    raise ValueError(w.kind)
