"""torch-facing wrappers over the W8A8 / SmoothQuant entry points of
libw4a16.so (`include/w8a8.h`): calibration maxima, smoothing factors,
per-channel INT8 weights, per-token INT8 activations and the int8 product.

Only argument marshalling happens here: tensors must already live on the GPU
and the library does all of the arithmetic on torch's current stream.
"""
from dataclasses import dataclass

import torch

from ._lib import W4A16Error, check, lib
from .api import _need, _same_device, _stream


def _dev(t, dtype, name):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise W4A16Error(f"{name} must be a GPU tensor (there is no CPU implementation)")
    if t.dtype != dtype:
        raise W4A16Error(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise W4A16Error(f"{name} must be contiguous")


def absmax_update(t, amax):
    """amax[j] = max(amax[j], max_r |t[r, j]|) for fp16 or fp32 t [rows, cols]."""
    if t.dim() != 2:
        raise W4A16Error("t must be 2-D [rows, cols]")
    fn = {torch.float16: "sq_absmax_update_f16", torch.float32: "sq_absmax_update_f32"}.get(t.dtype)
    if fn is None:
        raise W4A16Error("t must be float16 (activations) or float32 (weights)")
    _dev(t, t.dtype, "t")
    _need(amax, torch.float32, (t.shape[1],), "amax")
    _same_device(t, amax)
    with torch.cuda.device(t.device):
        check(getattr(lib(), fn)(t.data_ptr(), t.shape[0], t.shape[1], amax.data_ptr(), _stream(t)), fn)
    return amax


def smooth_factors(act_max, w_max, alpha=0.5, out=None):
    """s_j = max(act_max_j^alpha / max(w_max_j, 1e-5)^(1-alpha), 1e-5)."""
    _dev(act_max, torch.float32, "act_max")
    n = act_max.numel()
    _need(w_max, torch.float32, (n,), "w_max")
    out = torch.empty(n, dtype=torch.float32, device=act_max.device) if out is None else out
    _need(out, torch.float32, (n,), "out")
    _same_device(act_max, w_max, out)
    with torch.cuda.device(act_max.device):
        check(lib().sq_smooth_factors(act_max.data_ptr(), w_max.data_ptr(), n, float(alpha), out.data_ptr(),
                                      _stream(act_max)), "sq_smooth_factors")
    return out


def quantize_weight(w, s=None):
    """fp32 W [n_out, k] (times diag(s)) -> (int8 [n_out, k], fp32 scale [n_out])."""
    _dev(w, torch.float32, "w")
    n_out, k = w.shape
    if s is not None:
        _need(s, torch.float32, (k,), "s")
    qw = torch.empty((n_out, k), dtype=torch.int8, device=w.device)
    sw = torch.empty(n_out, dtype=torch.float32, device=w.device)
    with torch.cuda.device(w.device):
        check(lib().w8a8_quantize_weight(w.data_ptr(), None if s is None else s.data_ptr(), n_out, k,
                                         qw.data_ptr(), sw.data_ptr(), _stream(w)), "w8a8_quantize_weight")
    return qw, sw


def quantize_act(x, s=None, qx=None, sx=None):
    """fp16 x [m, k] (divided by s) -> (int8 [m, k], fp32 scale [m]), per token."""
    _dev(x, torch.float16, "x")
    m, k = x.shape
    if s is not None:
        _need(s, torch.float32, (k,), "s")
    qx = torch.empty((m, k), dtype=torch.int8, device=x.device) if qx is None else qx
    sx = torch.empty(m, dtype=torch.float32, device=x.device) if sx is None else sx
    _need(qx, torch.int8, (m, k), "qx")
    _need(sx, torch.float32, (m,), "sx")
    with torch.cuda.device(x.device):
        check(lib().w8a8_quantize_act(x.data_ptr(), None if s is None else s.data_ptr(), m, k, qx.data_ptr(),
                                      sx.data_ptr(), _stream(x)), "w8a8_quantize_act")
    return qx, sx


def gemm(qx, sx, qw, sw, out=None):
    """y fp16 [m, n_out] = fp16((acc * sx[m]) * sw[n]), acc the exact int8 product."""
    _dev(qx, torch.int8, "qx")
    _dev(qw, torch.int8, "qw")
    m, k = qx.shape
    n_out = qw.shape[0]
    _need(qw, torch.int8, (n_out, k), "qw")
    _need(sx, torch.float32, (m,), "sx")
    _need(sw, torch.float32, (n_out,), "sw")
    out = torch.empty((m, n_out), dtype=torch.float16, device=qx.device) if out is None else out
    _need(out, torch.float16, (m, n_out), "out")
    _same_device(qx, sx, qw, sw, out)
    with torch.cuda.device(qx.device):
        check(lib().w8a8_gemm(qx.data_ptr(), sx.data_ptr(), qw.data_ptr(), sw.data_ptr(), m, n_out, k,
                              out.data_ptr(), _stream(qx)), "w8a8_gemm")
    return out


@dataclass
class W8A8Linear:
    """A linear layer W [n_out, k] smoothed with s and quantized to INT8 per
    output channel; forward quantizes x / s per token and runs the int8 product."""
    qw: torch.Tensor
    sw: torch.Tensor
    s: torch.Tensor

    @classmethod
    def from_float(cls, w, act_max, alpha=0.5):
        w_max = torch.zeros(w.shape[1], dtype=torch.float32, device=w.device)
        absmax_update(w, w_max)
        s = smooth_factors(act_max, w_max, alpha)
        qw, sw = quantize_weight(w, s)
        return cls(qw, sw, s)

    def __call__(self, x, out=None):
        qx, sx = quantize_act(x, self.s)
        return gemm(qx, sx, self.qw, self.sw, out)
