"""The Python binding's own checks (transformer_attention_flash_amd/api.py):
shapes, dtypes, device and layout are validated before any library call, so
these run without a GPU.  The sizes the C ABI receives come from q's shape;
a tensor of another shape would be read or written out of bounds, so every
mismatch must raise here."""
import pytest
import torch

import transformer_attention_flash_amd as plx

BF = torch.bfloat16


def t(*shape, dtype=BF):
    return torch.zeros(shape, dtype=dtype)


def test_prefill_shape_checks():
    q, k = t(1, 4, 16, 64), t(1, 2, 16, 64)
    with pytest.raises(ValueError, match="4-D"):
        plx.prefill(t(4, 16, 64), k, k)
    with pytest.raises(ValueError, match="k and v"):
        plx.prefill(q, t(1, 2, 15, 64), t(1, 2, 15, 64))
    with pytest.raises(ValueError, match="k and v"):
        plx.prefill(q, k, t(1, 2, 16, 32))
    with pytest.raises(ValueError, match="rho"):
        plx.prefill(q, k, k, t(1, 4, 16, 32))
    with pytest.raises(ValueError, match="out"):
        plx.prefill(q, k, k, out=t(1, 4, 8, 64))
    with pytest.raises(ValueError, match="GPU tensor"):
        plx.prefill(q, k, k)


def test_dtype_checks():
    q, k = t(1, 4, 16, 64, dtype=torch.float16), t(1, 2, 16, 64, dtype=torch.float16)
    with pytest.raises(ValueError):
        plx.prefill(q, k, k)
    with pytest.raises(ValueError):
        plx.prefill(t(1, 4, 16, 64), t(1, 2, 16, 64, dtype=torch.float32), t(1, 2, 16, 64, dtype=torch.float32))


def test_prefill_backward_shape_checks():
    B, Hq, Hkv, T, d = 1, 4, 2, 16, 64
    q, k, lse = t(B, Hq, T, d), t(B, Hkv, T, d), t(B, Hq, T, dtype=torch.float32)
    good = dict(q=q, k=k, v=k, rho=q, out=q, out_sa=q, lse=lse, rbar=lse, dout=q)

    def call(**over):
        a = dict(good, **over)
        return plx.prefill_backward(a["q"], a["k"], a["v"], a["rho"], a["out"], a["out_sa"], a["lse"], a["rbar"],
                                    a["dout"])
    with pytest.raises(ValueError, match="lse"):
        call(lse=t(B, Hq, dtype=torch.float32))
    with pytest.raises(ValueError, match="rbar"):
        call(rbar=t(B, Hq, T + 1, dtype=torch.float32))
    with pytest.raises(ValueError, match="out_sa"):
        call(out_sa=t(B, Hq, T, d + 1))
    with pytest.raises(ValueError, match="dout"):
        call(dout=t(B, Hq, T - 1, d))
    with pytest.raises(ValueError, match="k and v"):
        call(v=t(B, Hkv, T, d + 64))
    with pytest.raises(ValueError, match="lse is required"):
        call(lse=None)
    with pytest.raises(ValueError, match="GPU tensor"):
        call()


def test_decode_shape_checks():
    q, kc = t(2, 4, 64), t(2, 2, 100, 64)
    with pytest.raises(ValueError, match="q must be"):
        plx.decode(t(2, 4, 1, 64), kc, kc)
    with pytest.raises(ValueError, match="contiguous k_cache"):
        plx.decode(q, t(3, 2, 100, 64), t(3, 2, 100, 64))
    with pytest.raises(ValueError, match="max_ctx"):
        plx.decode(q, kc, kc, max_ctx=50)
    with pytest.raises(ValueError, match="ragged"):
        plx.decode(q, t(500), t(500), cu_seqlens=torch.zeros(3, dtype=torch.int64))
    with pytest.raises(ValueError, match="cu_seqlens"):
        plx.decode(q, t(500), t(500), cu_seqlens=torch.zeros(3, dtype=torch.int32), num_kv_heads=2, max_ctx=10)
    with pytest.raises(ValueError, match="rho"):
        plx.decode(q, kc, kc, t(2, 4, 32))
    with pytest.raises(ValueError, match="out"):
        plx.decode(q, kc, kc, out=t(2, 4, 32))
    with pytest.raises(ValueError, match="GPU tensor"):
        plx.decode(q, kc, kc)


def test_projection_shape_checks():
    with pytest.raises(ValueError, match="x must be"):
        plx.qkvr_projection(t(8, 64), t(6 * 64, 64), 2, 1, 64)
    with pytest.raises(ValueError, match="w must be"):
        plx.qkvr_projection(t(1, 8, 64), t(5 * 64, 64), 2, 1, 64)
    with pytest.raises(ValueError, match="GPU tensor"):
        plx.qkvr_projection(t(1, 8, 64), t(6 * 64, 64), 2, 1, 64)


class _FakeGpuTensor:
    """Stands in for a GPU tensor on a machine without one: only the
    attributes the binding's checks read."""

    def __init__(self, index, dtype=BF):
        self.is_cuda = True
        self.dtype = dtype
        self.device = torch.device("cuda", index)

    def is_contiguous(self):
        return True


def test_tensors_on_two_devices_are_rejected():
    from transformer_attention_flash_amd import api
    a, b = _FakeGpuTensor(0), _FakeGpuTensor(1)
    with pytest.raises(ValueError, match="other tensors are on cuda:0"):
        api._check_tensors(BF, q=a, k=b)
    with pytest.raises(ValueError, match="workspace is on cuda:1"):
        api._check_device(q=a, workspace=b)
    api._check_device(q=a, k=_FakeGpuTensor(0), rho=None)  # one device: accepted
