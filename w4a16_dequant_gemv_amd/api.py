"""torch-facing wrappers over the C ABI of libw4a16.so.

Only argument marshalling happens here: tensors must already live on the GPU;
their data pointers and torch's current HIP stream are handed to the library,
which does all of the arithmetic.  There is no CPU path.
"""
from dataclasses import dataclass

import torch

from ._lib import W4A16Error, check, lib

GROUP_SIZES = (32, 64, 128, 256)
BITS = (4, 8)
MAX_GEMV_ROWS = 16


@dataclass
class QuantizedWeight:
    """Packed INT4 (bits=4) or INT8 (bits=8) weight of a linear layer W[n_out, n_in].

    qweight: int32 [n_out, n_in * bits // 32]; element k of a row is the code
             in bits bits*(k % (32/bits)).. of word k // (32/bits) (the int32
             holds the u32 bits).
    scales, zeros: float16 [n_out, n_in // group_size]; w' = s * (code - z).
    group_size == n_in is one scale per output channel.
    """
    qweight: torch.Tensor
    scales: torch.Tensor
    zeros: torch.Tensor
    n_out: int
    n_in: int
    group_size: int
    symmetric: bool = False
    bits: int = 4

    def nbytes(self):
        return (self.qweight.numel() * 4 + self.scales.numel() * 2 + self.zeros.numel() * 2)


def _stream(t):
    """Handle of torch's current HIP stream on t's device."""
    return torch.cuda.current_stream(t.device).cuda_stream


def _need(t, dtype, shape, name):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise W4A16Error(f"{name} must be a GPU tensor (there is no CPU implementation)")
    if t.dtype != dtype:
        raise W4A16Error(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise W4A16Error(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise W4A16Error(f"{name} must be contiguous")


def _same_device(*ts):
    d = ts[0].device
    for t in ts[1:]:
        if t.device != d:
            raise W4A16Error("all tensors must be on the same GPU")


def _prefix(bits):
    if bits not in BITS:
        raise W4A16Error(f"bits must be one of {BITS}, got {bits}")
    return f"q{bits}_"


def quantize_pack(w, group_size=128, symmetric=False, out=None, bits=4):
    """fp32 W [n_out, n_in] on the GPU -> QuantizedWeight (bit-exact INT4 or INT8).
    group_size None (or n_in) quantizes per output channel."""
    if w.dim() != 2:
        raise W4A16Error("w must be 2-D [n_out, n_in]")
    n_out, n_in = w.shape
    if group_size is None:
        group_size = n_in
    per_channel = group_size == n_in and n_in % 32 == 0
    if (group_size not in GROUP_SIZES and not per_channel) or n_in % group_size:
        raise W4A16Error(f"group_size {group_size} must be one of {GROUP_SIZES} (dividing n_in={n_in}) "
                         f"or n_in itself with n_in % 32 == 0")
    prefix = _prefix(bits)
    _need(w, torch.float32, (n_out, n_in), "w")
    G = n_in // group_size
    words = n_in * bits // 32
    if out is None:
        out = QuantizedWeight(
            torch.empty((n_out, words), dtype=torch.int32, device=w.device),
            torch.empty((n_out, G), dtype=torch.float16, device=w.device),
            torch.empty((n_out, G), dtype=torch.float16, device=w.device),
            n_out, n_in, group_size, bool(symmetric), bits)
    else:
        _need(out.qweight, torch.int32, (n_out, words), "out.qweight")
        _need(out.scales, torch.float16, (n_out, G), "out.scales")
        _need(out.zeros, torch.float16, (n_out, G), "out.zeros")
        out.group_size, out.symmetric, out.bits = group_size, bool(symmetric), bits
    _same_device(w, out.qweight, out.scales, out.zeros)
    with torch.cuda.device(w.device):
        check(getattr(lib(), prefix + "quantize_pack")(
            w.data_ptr(), n_out, n_in, group_size, int(bool(symmetric)), out.qweight.data_ptr(),
            out.scales.data_ptr(), out.zeros.data_ptr(), _stream(w)), prefix + "quantize_pack")
    return out


def _check_qw(qw):
    _prefix(qw.bits)
    _need(qw.qweight, torch.int32, (qw.n_out, qw.n_in * qw.bits // 32), "qweight")
    G = qw.n_in // qw.group_size
    _need(qw.scales, torch.float16, (qw.n_out, G), "scales")
    _need(qw.zeros, torch.float16, (qw.n_out, G), "zeros")


def dequant(qw, out=None):
    """QuantizedWeight (INT4 or INT8) -> fp32 W' [n_out, n_in], w' = s * (code - z), bit-exact."""
    _check_qw(qw)
    dev = qw.qweight.device
    if out is None:
        out = torch.empty((qw.n_out, qw.n_in), dtype=torch.float32, device=dev)
    _need(out, torch.float32, (qw.n_out, qw.n_in), "out")
    _same_device(qw.qweight, qw.scales, qw.zeros, out)
    name = _prefix(qw.bits) + "dequant"
    with torch.cuda.device(dev):
        check(getattr(lib(), name)(qw.qweight.data_ptr(), qw.scales.data_ptr(), qw.zeros.data_ptr(),
                                   qw.n_out, qw.n_in, qw.group_size, out.data_ptr(), _stream(out)),
              name)
    return out


def _linear(kind, x, qw, out):
    _check_qw(qw)
    fn_name = _prefix(qw.bits) + kind
    if x.dim() != 2:
        raise W4A16Error("x must be 2-D [m, n_in]")
    m = x.shape[0]
    _need(x, torch.float16, (m, qw.n_in), "x")
    if out is None:
        out = torch.empty((m, qw.n_out), dtype=torch.float16, device=x.device)
    _need(out, torch.float16, (m, qw.n_out), "out")
    if m == 0:
        return out          # an empty batch has nothing to compute
    _same_device(x, qw.qweight, qw.scales, qw.zeros, out)
    with torch.cuda.device(x.device):
        check(getattr(lib(), fn_name)(x.data_ptr(), qw.qweight.data_ptr(), qw.scales.data_ptr(),
                                      qw.zeros.data_ptr(), m, qw.n_out, qw.n_in, qw.group_size,
                                      out.data_ptr(), _stream(x)), fn_name)
    return out


def gemv(x, qw, out=None):
    """Decode-shaped y = x W'^T, x fp16 [m <= 16, n_in] -> y fp16 [m, n_out]."""
    return _linear("gemv", x, qw, out)


def gemm(x, qw, out=None):
    """Prefill-shaped y = x W'^T for any m, tuned for large m."""
    return _linear("gemm", x, qw, out)


def kernel_config(kind, bits, m, n_out, n_in, group_size, scales_ptr=256, zeros_ptr=256):
    """Name of the kernel instantiation gemv (kind "gemv") or gemm (kind
    "gemm") launches for these sizes, as profilers print it.  Nothing is
    launched; works without a GPU.  The selection can depend on the alignment
    of the scale and zero-point arrays: pass their data_ptr() values (the
    default, 256, stands for freshly allocated arrays)."""
    import ctypes
    if kind not in ("gemv", "gemm"):
        raise W4A16Error(f"kind must be 'gemv' or 'gemm', got {kind!r}")
    if group_size is None:
        group_size = n_in
    buf = ctypes.create_string_buffer(128)
    check(lib().q4_linear_config(0 if kind == "gemv" else 1, bits, m, n_out, n_in, group_size,
                                 scales_ptr, zeros_ptr, buf, len(buf)), "q4_linear_config")
    return buf.value.decode()


def linear(x, qw, out=None):
    """y = x W'^T, routed to the GEMV kernels for m <= 16 and the GEMM otherwise."""
    return gemv(x, qw, out) if x.shape[0] <= MAX_GEMV_ROWS else gemm(x, qw, out)
