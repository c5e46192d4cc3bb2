"""torch-facing wrappers over the KV-cache codec of libw4a16.so
(`include/kv_codec.h`): V quantized per token, K per channel over blocks of
tokens, symmetric INT8 or INT4 codes in int8, fp32 scales.

Only argument marshalling happens here: tensors must already live on the GPU
and the library does all of the arithmetic on torch's current stream.
"""
import torch

from ._lib import W4A16Error, check, lib
from .api import _need, _same_device, _stream


def _dev_tensor(t, dtype, name):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise W4A16Error(f"{name} must be a GPU tensor (there is no CPU implementation)")
    if t.dtype != dtype:
        raise W4A16Error(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise W4A16Error(f"{name} must be contiguous")


def quant_tokens(x, bits=8, q=None, scale=None):
    """fp16 x [..., d] -> (int8 q [..., d], fp32 scale [...]): one symmetric
    scale per token row over the head dimension (the V side)."""
    _dev_tensor(x, torch.float16, "x")
    d = x.shape[-1]
    rows = x.numel() // d
    q = torch.empty(x.shape, dtype=torch.int8, device=x.device) if q is None else q
    scale = torch.empty(x.shape[:-1], dtype=torch.float32, device=x.device) if scale is None else scale
    _need(q, torch.int8, x.shape, "q")
    _need(scale, torch.float32, x.shape[:-1], "scale")
    _same_device(x, q, scale)
    with torch.cuda.device(x.device):
        check(lib().kv_quant_tokens(x.data_ptr(), rows, d, bits, q.data_ptr(), scale.data_ptr(), _stream(x)),
              "kv_quant_tokens")
    return q, scale


def quant_channels(x, bits=8, q=None, scale=None):
    """fp16 x [blocks, t, d] -> (int8 q [blocks, t, d], fp32 scale [blocks, d]):
    one symmetric scale per channel of each block of t tokens (the K side)."""
    _dev_tensor(x, torch.float16, "x")
    if x.dim() != 3:
        raise W4A16Error("x must be [blocks, t, d]")
    blocks, t, d = x.shape
    q = torch.empty(x.shape, dtype=torch.int8, device=x.device) if q is None else q
    scale = torch.empty((blocks, d), dtype=torch.float32, device=x.device) if scale is None else scale
    _need(q, torch.int8, x.shape, "q")
    _need(scale, torch.float32, (blocks, d), "scale")
    _same_device(x, q, scale)
    with torch.cuda.device(x.device):
        check(lib().kv_quant_channels(x.data_ptr(), blocks, t, d, bits, q.data_ptr(), scale.data_ptr(),
                                      _stream(x)), "kv_quant_channels")
    return q, scale


def dequant_tokens(q, scale, out=None):
    """int8 q [..., d], fp32 scale [...] -> fp16 q * scale."""
    _dev_tensor(q, torch.int8, "q")
    d = q.shape[-1]
    _need(scale, torch.float32, q.shape[:-1], "scale")
    out = torch.empty(q.shape, dtype=torch.float16, device=q.device) if out is None else out
    _need(out, torch.float16, q.shape, "out")
    _same_device(q, scale, out)
    with torch.cuda.device(q.device):
        check(lib().kv_dequant_tokens(q.data_ptr(), scale.data_ptr(), q.numel() // d, d, out.data_ptr(),
                                      _stream(q)), "kv_dequant_tokens")
    return out


def dequant_channels(q, scale, out=None):
    """int8 q [blocks, t, d], fp32 scale [blocks, d] -> fp16 q * scale."""
    _dev_tensor(q, torch.int8, "q")
    if q.dim() != 3:
        raise W4A16Error("q must be [blocks, t, d]")
    blocks, t, d = q.shape
    _need(scale, torch.float32, (blocks, d), "scale")
    out = torch.empty(q.shape, dtype=torch.float16, device=q.device) if out is None else out
    _need(out, torch.float16, q.shape, "out")
    _same_device(q, scale, out)
    with torch.cuda.device(q.device):
        check(lib().kv_dequant_channels(q.data_ptr(), scale.data_ptr(), blocks, t, d, out.data_ptr(),
                                        _stream(q)), "kv_dequant_channels")
    return out


class KVBlockPool:
    """A pool of quantized KV blocks of t tokens x d channels for one layer's
    heads: K codes with per-channel scales, V codes with per-token scales."""

    def __init__(self, pool_blocks, t, d, device, bits=8):
        self.t, self.d, self.bits = t, d, bits
        self.k = torch.zeros((pool_blocks, t, d), dtype=torch.int8, device=device)
        self.k_scale = torch.zeros((pool_blocks, d), dtype=torch.float32, device=device)
        self.v = torch.zeros((pool_blocks, t, d), dtype=torch.int8, device=device)
        self.v_scale = torch.zeros((pool_blocks, t), dtype=torch.float32, device=device)

    @property
    def pool_blocks(self):
        return self.k.shape[0]

    def flush(self, k_blocks, v_blocks, dst):
        """Quantize fp16 window blocks k_blocks / v_blocks [P, t, d] into the
        slots dst (int32 [P] on the GPU); slots outside the pool are skipped."""
        for name, tns in (("k_blocks", k_blocks), ("v_blocks", v_blocks)):
            _dev_tensor(tns, torch.float16, name)
        P = k_blocks.shape[0]
        _need(v_blocks, torch.float16, (P, self.t, self.d), "v_blocks")
        _need(k_blocks, torch.float16, (P, self.t, self.d), "k_blocks")
        _need(dst, torch.int32, (P,), "dst")
        _same_device(k_blocks, v_blocks, dst, self.k)
        with torch.cuda.device(self.k.device):
            check(lib().kv_flush_blocks(k_blocks.data_ptr(), v_blocks.data_ptr(), P, self.t, self.d, self.bits,
                                        dst.data_ptr(), self.pool_blocks, self.k.data_ptr(),
                                        self.k_scale.data_ptr(), self.v.data_ptr(), self.v_scale.data_ptr(),
                                        _stream(self.k)), "kv_flush_blocks")
