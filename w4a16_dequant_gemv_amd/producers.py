"""torch-facing wrappers over GPTQ and AWQ in libw4a16.so (`include/producers.h`):
calibration-driven producers of the packed weights that `quantize_pack` writes.

Only argument marshalling happens here (including the device workspace the
library asks for); the arithmetic runs in the library on torch's current stream.
"""
import torch

from ._lib import W4A16Error, check, lib
from .api import QuantizedWeight, _need, _same_device, _stream


def _dev(t, dtype, name):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise W4A16Error(f"{name} must be a GPU tensor (there is no CPU implementation)")
    if t.dtype != dtype:
        raise W4A16Error(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise W4A16Error(f"{name} must be contiguous")


def _workspace(nbytes, device):
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def _outputs(n_out, n, group_size, bits, symmetric, device):
    G = n // group_size
    return QuantizedWeight(torch.empty((n_out, n * bits // 32), dtype=torch.int32, device=device),
                           torch.empty((n_out, G), dtype=torch.float16, device=device),
                           torch.empty((n_out, G), dtype=torch.float16, device=device),
                           n_out, n, group_size, bool(symmetric), bits)


def gptq_factor(x, damp=0.01):
    """fp16 calibration tokens x [tokens, n] -> fp32 U [n, n], the upper
    Cholesky factor of (2 x^T x + damp * mean(diag) I)^-1."""
    _dev(x, torch.float16, "x")
    tokens, n = x.shape
    ws = _workspace(lib().gptq_factor_workspace_size(n), x.device)
    u = torch.empty((n, n), dtype=torch.float32, device=x.device)
    with torch.cuda.device(x.device):
        check(lib().gptq_hinv_factor(x.data_ptr(), tokens, n, float(damp), ws.data_ptr(), ws.numel(), u.data_ptr(),
                                     _stream(x)), "gptq_hinv_factor")
    return u


def gptq_quantize(w, u, group_size=128, bits=4, symmetric=False):
    """The GPTQ column loop on fp32 W [n_out, n] with the factor U."""
    _dev(w, torch.float32, "w")
    n_out, n = w.shape
    _need(u, torch.float32, (n, n), "u")
    _same_device(w, u)
    if group_size is None:
        group_size = n
    qw = _outputs(n_out, n, group_size, bits, symmetric, w.device)
    ws = _workspace(lib().gptq_quantize_workspace_size(n_out, n), w.device)
    with torch.cuda.device(w.device):
        check(lib().gptq_quantize(w.data_ptr(), u.data_ptr(), n_out, n, group_size, bits, int(bool(symmetric)),
                                  ws.data_ptr(), ws.numel(), qw.qweight.data_ptr(), qw.scales.data_ptr(),
                                  qw.zeros.data_ptr(), _stream(w)), "gptq_quantize")
    return qw


def gptq_quantize_noalloc(w, u, group_size=128, bits=4, symmetric=False, out=None):
    """gptq_quantize through the entry point that allocates nothing on the
    device (its scratch is the library's own fixed array); pass `out` (a
    QuantizedWeight) to make the call allocation-free on the torch side too."""
    _dev(w, torch.float32, "w")
    n_out, n = w.shape
    _need(u, torch.float32, (n, n), "u")
    _same_device(w, u)
    if group_size is None:
        group_size = n
    qw = out if out is not None else _outputs(n_out, n, group_size, bits, symmetric, w.device)
    with torch.cuda.device(w.device):
        check(lib().gptq_quantize_noalloc(w.data_ptr(), u.data_ptr(), n_out, n, group_size, bits,
                                          int(bool(symmetric)), qw.qweight.data_ptr(), qw.scales.data_ptr(),
                                          qw.zeros.data_ptr(), _stream(w)), "gptq_quantize_noalloc")
    return qw


def gptq(w, x, group_size=128, bits=4, symmetric=False, damp=0.01):
    """GPTQ of W [n_out, n] on calibration tokens x [tokens, n] -> QuantizedWeight."""
    return gptq_quantize(w, gptq_factor(x, damp), group_size, bits, symmetric)


def awq(w, x, group_size=128, bits=4, symmetric=False, n_grid=20):
    """AWQ of W [n_out, n] on calibration tokens x -> (QuantizedWeight, s [n]
    to divide the activations by, winning grid index, errors [n_grid + 1])."""
    _dev(w, torch.float32, "w")
    _dev(x, torch.float16, "x")
    n_out, n = w.shape
    tokens = x.shape[0]
    if x.shape[1] != n:
        raise W4A16Error("x must be [tokens, n] with the weight's n")
    if group_size is None:
        group_size = n
    qw = _outputs(n_out, n, group_size, bits, symmetric, w.device)
    s = torch.empty(n, dtype=torch.float32, device=w.device)
    best = torch.empty(1, dtype=torch.int32, device=w.device)
    losses = torch.empty(n_grid + 1, dtype=torch.float32, device=w.device)
    ws = _workspace(lib().awq_workspace_size(n_out, n, tokens, n_grid, group_size), w.device)
    with torch.cuda.device(w.device):
        check(lib().awq_quantize(w.data_ptr(), x.data_ptr(), tokens, n_out, n, group_size, bits, int(bool(symmetric)),
                                 n_grid, ws.data_ptr(), ws.numel(), qw.qweight.data_ptr(), qw.scales.data_ptr(),
                                 qw.zeros.data_ptr(), s.data_ptr(), best.data_ptr(), losses.data_ptr(), _stream(w)),
              "awq_quantize")
    return qw, s, best, losses
