"""Python entry points over libparallax.so.

These functions only marshal arguments: they check that the tensors are on
the GPU, contiguous and of one dtype, allocate the output (and the decode
workspace) with torch, and pass raw device pointers and torch's current
stream to the C ABI.  Every step of the computation runs in the HIP kernels.
"""
from __future__ import annotations

import math
from typing import Optional

import torch

from . import _native as N

_DTYPES = {torch.bfloat16: N.PLX_DTYPE_BF16, torch.float32: N.PLX_DTYPE_F32}


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    dev = getattr(stream, "device", None)
    if dev is not None and dev.index is not None and dev.index != torch.cuda.current_device():
        raise ValueError(f"stream belongs to {dev} but the current device is cuda:{torch.cuda.current_device()}")
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _check_device(**tensors):
    """All given GPU tensors on one device, and that device the current one:
    the kernels launch on the current device's stream, which must be able to
    address every pointer."""
    dev = None
    for name, t in tensors.items():
        if t is None:
            continue
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"{name} is on {t.device}, the other tensors are on {dev}")
    if dev is not None and dev.index is not None and torch.cuda.is_available() \
            and dev.index != torch.cuda.current_device():
        raise ValueError(f"the tensors are on {dev} but the current device is cuda:{torch.cuda.current_device()}; "
                         f"call under torch.cuda.device({dev.index})")


def _check_tensors(dtype, **tensors):
    for name, t in tensors.items():
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if t.dtype != dtype:
            raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    _check_device(**tensors)


def _dtype_code(dtype) -> int:
    if dtype not in _DTYPES:
        raise ValueError(f"unsupported dtype {dtype}; use bfloat16 or float32")
    return _DTYPES[dtype]


def prefill(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, rho: Optional[torch.Tensor] = None, *,
            scale: Optional[float] = None, out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Causal Parallax prefill.  q, rho: [B, Hq, T, d]; k, v: [B, Hkv, T, d].

    rho=None runs the softmax-only kernel.  scale defaults to 1/sqrt(d).
    """
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q and k must be 4-D [B, H, T, d]")
    B, Hq, T, d = q.shape
    Hkv = k.shape[1]
    if k.shape != (B, Hkv, T, d) or v.shape != k.shape:
        raise ValueError("k and v must be [B, Hkv, T, d] matching q")
    if rho is not None and rho.shape != q.shape:
        raise ValueError("rho must have q's shape")
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape:
        raise ValueError("out must have q's shape")
    _check_tensors(q.dtype, q=q, k=k, v=v, rho=rho, out=out)
    code = _dtype_code(q.dtype)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    st = N.load().parallax_fwd_prefill(_ptr(q), _ptr(k), _ptr(v), _ptr(rho), _ptr(out), B, Hq, Hkv, T, d,
                                       scale, code, _stream(stream))
    N.check(st, "parallax_fwd_prefill")
    return out


def prefill_train(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, rho: Optional[torch.Tensor] = None, *,
                  scale: Optional[float] = None, stream=None):
    """Causal Parallax prefill that also keeps what the backward needs (bf16).

    Returns (out, out_sa, lse, rbar): out and out_sa shaped like q; lse and
    rbar fp32 [B, Hq, T] (lse in log2 units); out_sa and rbar are None
    without rho.
    """
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q and k must be 4-D [B, H, T, d]")
    B, Hq, T, d = q.shape
    Hkv = k.shape[1]
    if k.shape != (B, Hkv, T, d) or v.shape != k.shape:
        raise ValueError("k and v must be [B, Hkv, T, d] matching q")
    if rho is not None and rho.shape != q.shape:
        raise ValueError("rho must have q's shape")
    _check_tensors(q.dtype, q=q, k=k, v=v, rho=rho)
    code = _dtype_code(q.dtype)
    out = torch.empty_like(q)
    out_sa = None if rho is None else torch.empty_like(q)
    lse = torch.empty((B, Hq, T), dtype=torch.float32, device=q.device)
    rbar = None if rho is None else torch.empty((B, Hq, T), dtype=torch.float32, device=q.device)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    st = N.load().parallax_fwd_prefill_train(_ptr(q), _ptr(k), _ptr(v), _ptr(rho), _ptr(out), _ptr(out_sa),
                                             _ptr(lse), _ptr(rbar), B, Hq, Hkv, T, d, scale, code,
                                             _stream(stream))
    N.check(st, "parallax_fwd_prefill_train")
    return out, out_sa, lse, rbar


def prefill_backward(q, k, v, rho, out, out_sa, lse, rbar, dout, *, scale: Optional[float] = None,
                     workspace: Optional[torch.Tensor] = None, stream=None):
    """Gradients (dq, dk, dv, drho) of sum(dout * out) for the causal Parallax
    prefill, from the tensors prefill_train returned (bf16).  drho is None
    when rho is."""
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q and k must be 4-D [B, H, T, d]")
    B, Hq, T, d = q.shape
    Hkv = k.shape[1]
    if k.shape != (B, Hkv, T, d) or v.shape != k.shape:
        raise ValueError("k and v must be [B, Hkv, T, d] matching q")
    for name, t in (("out", out), ("dout", dout), ("rho", rho), ("out_sa", out_sa)):
        if t is not None and t.shape != q.shape:
            raise ValueError(f"{name} must have q's shape")
    for name, t in (("lse", lse), ("rbar", rbar)):
        if t is not None and t.shape != (B, Hq, T):
            raise ValueError(f"{name} must be [B, Hq, T]")
    if lse is None:
        raise ValueError("lse is required")
    _check_tensors(q.dtype, q=q, k=k, v=v, rho=rho, out=out, out_sa=out_sa, dout=dout)
    _check_tensors(torch.float32, lse=lse, rbar=rbar)
    code = _dtype_code(q.dtype)
    lib = N.load()
    need = lib.parallax_bwd_prefill_workspace_size(B, Hq, T)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    elif not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous GPU tensor")
    _check_device(q=q, lse=lse, workspace=workspace)
    dq = torch.empty_like(q)
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    drho = None if rho is None else torch.empty_like(q)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    st = lib.parallax_bwd_prefill(_ptr(q), _ptr(k), _ptr(v), _ptr(rho), _ptr(out), _ptr(out_sa), _ptr(lse),
                                  _ptr(rbar), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(drho),
                                  B, Hq, Hkv, T, d, scale, code, _ptr(workspace),
                                  workspace.numel() * workspace.element_size(), _stream(stream))
    N.check(st, "parallax_bwd_prefill")
    return dq, dk, dv, drho


class ParallaxAttention(torch.autograd.Function):
    """torch.autograd wrapper: forward = prefill_train, backward =
    prefill_backward (bf16, causal).  Marshalling only."""

    @staticmethod
    def forward(ctx, q, k, v, rho, scale):
        out, out_sa, lse, rbar = prefill_train(q, k, v, rho, scale=scale)
        ctx.save_for_backward(q, k, v, rho, out, out_sa, lse, rbar)
        ctx.scale = scale
        return out

    @staticmethod
    def backward(ctx, dout):
        q, k, v, rho, out, out_sa, lse, rbar = ctx.saved_tensors
        dq, dk, dv, drho = prefill_backward(q, k, v, rho, out, out_sa, lse, rbar, dout.contiguous(),
                                            scale=ctx.scale)
        return dq, dk, dv, drho, None


def qkvr_projection(x: torch.Tensor, w: torch.Tensor, Hq: int, Hkv: int, d: int, *, stream=None):
    """Fused q/k/v/probe projection.  x: [B, T, d_model]; w: [(2 Hq + 2 Hkv) d,
    d_model] (q, k, v, probe rows).  Returns (q, k, v, rho) in the attention
    layout [B, H, T, d] (bf16)."""
    if x.dim() != 3:
        raise ValueError("x must be [B, T, d_model]")
    B, T, dm = x.shape
    if w.shape != ((2 * Hq + 2 * Hkv) * d, dm):
        raise ValueError("w must be [(2 Hq + 2 Hkv) d, d_model]")
    _check_tensors(x.dtype, x=x, w=w)
    code = _dtype_code(x.dtype)
    q = torch.empty((B, Hq, T, d), dtype=x.dtype, device=x.device)
    k = torch.empty((B, Hkv, T, d), dtype=x.dtype, device=x.device)
    v = torch.empty_like(k)
    rho = torch.empty_like(q)
    st = N.load().parallax_qkvr_projection(_ptr(x), _ptr(w), _ptr(q), _ptr(k), _ptr(v), _ptr(rho), B, T, dm, Hq,
                                           Hkv, d, code, _stream(stream))
    N.check(st, "parallax_qkvr_projection")
    return q, k, v, rho


def decode_workspace_size(B: int, Hq: int, Hkv: int, d: int, max_ctx: int, dtype=torch.bfloat16,
                          keys_per_split: int = 0) -> int:
    """Workspace bytes of a decode call: parallax_fwd_decode_workspace_size, or
    with keys_per_split != 0 parallax_fwd_decode_chunked_workspace_size."""
    lib = N.load()
    if keys_per_split:
        n = lib.parallax_fwd_decode_chunked_workspace_size(B, Hq, Hkv, d, int(max_ctx), _dtype_code(dtype),
                                                           int(keys_per_split))
    else:
        n = lib.parallax_fwd_decode_workspace_size(B, Hq, Hkv, d, int(max_ctx), _dtype_code(dtype))
    if n == (1 << 64) - 1:
        raise N.ParallaxError(N.PLX_ERR_INVALID_ARGUMENT, "parallax_fwd_decode_workspace_size")
    return int(n)


def decode_auto_split(B: int, Hq: int, Hkv: int, d: int, max_ctx: int) -> int:
    ks = N.load().parallax_fwd_decode_auto_split(B, Hq, Hkv, d, int(max_ctx))
    if ks < 0:
        raise N.ParallaxError(-ks, "parallax_fwd_decode_auto_split")
    return int(ks)


def _decode_args(q, k_cache, v_cache, rho, cu_seqlens, max_ctx, num_kv_heads, scale, out):
    """Shape checks shared by the decode entry points; returns the marshalled
    sizes and the output tensor."""
    if q.dim() != 3:
        raise ValueError("q must be [B, Hq, d]")
    B, Hq, d = q.shape
    if cu_seqlens is None:
        if k_cache.dim() != 4 or k_cache.shape[0] != B or k_cache.shape[3] != d:
            raise ValueError("contiguous k_cache must be [B, Hkv, L, d]")
        Hkv, L = k_cache.shape[1], k_cache.shape[2]
        if max_ctx is not None and max_ctx != L:
            raise ValueError("max_ctx must equal the cache length for a contiguous cache")
        max_ctx = L
    else:
        if num_kv_heads is None or max_ctx is None:
            raise ValueError("a ragged cache needs num_kv_heads and max_ctx")
        Hkv = int(num_kv_heads)
        if cu_seqlens.dtype != torch.int64 or cu_seqlens.shape != (B + 1,) or not cu_seqlens.is_cuda:
            raise ValueError("cu_seqlens must be a GPU int64 tensor of B + 1 offsets")
        if not cu_seqlens.is_contiguous():
            raise ValueError("cu_seqlens must be contiguous")
    if k_cache.shape != v_cache.shape:
        raise ValueError("k_cache and v_cache differ in shape")
    if rho is not None and rho.shape != q.shape:
        raise ValueError("rho must have q's shape")
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape:
        raise ValueError("out must have q's shape")
    _check_tensors(q.dtype, q=q, rho=rho, k_cache=k_cache, v_cache=v_cache, out=out)
    _check_device(q=q, cu_seqlens=cu_seqlens)
    code = _dtype_code(q.dtype)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    return B, Hq, Hkv, d, int(max_ctx), out, code, scale


def decode(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, rho: Optional[torch.Tensor] = None, *,
           cu_seqlens: Optional[torch.Tensor] = None, max_ctx: Optional[int] = None,
           num_kv_heads: Optional[int] = None, scale: Optional[float] = None, keys_per_split: int = 0,
           workspace: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
           stream=None) -> torch.Tensor:
    """Parallax decode: one query token per sequence.  q, rho: [B, Hq, d].

    Contiguous cache: k_cache, v_cache [B, Hkv, L, d] (cu_seqlens None).
    Ragged cache: cu_seqlens int64 [B + 1] on the GPU, k_cache / v_cache the
    packed slabs (any shape, contiguous), num_kv_heads and max_ctx required.
    keys_per_split=0 calls parallax_fwd_decode (the library chooses the
    chunking); any other value calls parallax_fwd_decode_chunked with it.
    """
    B, Hq, Hkv, d, max_ctx, out, code, scale = _decode_args(q, k_cache, v_cache, rho, cu_seqlens, max_ctx,
                                                            num_kv_heads, scale, out)
    need = decode_workspace_size(B, Hq, Hkv, d, max_ctx, q.dtype, keys_per_split)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    elif workspace is not None and (not workspace.is_cuda or not workspace.is_contiguous()):
        raise ValueError("workspace must be a contiguous GPU tensor")
    _check_device(q=q, workspace=workspace)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    lib = N.load()
    args = (_ptr(q), _ptr(rho), _ptr(k_cache), _ptr(v_cache), _ptr(cu_seqlens), max_ctx, _ptr(out), B, Hq,
            Hkv, d, scale, code)
    if keys_per_split:
        st = lib.parallax_fwd_decode_chunked(*args, int(keys_per_split), _ptr(workspace), ws_bytes,
                                             _stream(stream))
        N.check(st, "parallax_fwd_decode_chunked")
    else:
        st = lib.parallax_fwd_decode(*args, _ptr(workspace), ws_bytes, _stream(stream))
        N.check(st, "parallax_fwd_decode")
    return out


def decode_noalloc(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                   rho: Optional[torch.Tensor] = None, *, cu_seqlens: Optional[torch.Tensor] = None,
                   max_ctx: Optional[int] = None, num_kv_heads: Optional[int] = None,
                   scale: Optional[float] = None, out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """parallax_fwd_decode_noalloc: decode whose split partials go to the
    library's own per-device scratch, so the call allocates nothing (pass
    `out` to allocate nothing here either).  Arguments as decode()."""
    B, Hq, Hkv, d, max_ctx, out, code, scale = _decode_args(q, k_cache, v_cache, rho, cu_seqlens, max_ctx,
                                                            num_kv_heads, scale, out)
    st = N.load().parallax_fwd_decode_noalloc(_ptr(q), _ptr(rho), _ptr(k_cache), _ptr(v_cache), _ptr(cu_seqlens),
                                              max_ctx, _ptr(out), B, Hq, Hkv, d, scale, code, _stream(stream))
    N.check(st, "parallax_fwd_decode_noalloc")
    return out


# The C entry points' own names, for callers who think in terms of the ABI.
parallax_fwd_prefill = prefill
parallax_fwd_prefill_train = prefill_train
parallax_bwd_prefill = prefill_backward
parallax_qkvr_projection = qkvr_projection
parallax_fwd_decode = decode
parallax_fwd_decode_workspace_size = decode_workspace_size
parallax_fwd_decode_auto_split = decode_auto_split
parallax_fwd_decode_noalloc = decode_noalloc


def parallax_fwd_decode_chunked(q, k_cache, v_cache, rho=None, *, keys_per_split: int, **kw):
    """parallax_fwd_decode_chunked: decode with the caller's chunk size."""
    if keys_per_split <= 0:
        raise ValueError("keys_per_split must be positive (0 is parallax_fwd_decode's own choice)")
    return decode(q, k_cache, v_cache, rho, keys_per_split=keys_per_split, **kw)
