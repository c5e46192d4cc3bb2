"""Helpers shared by the GPU parity tests (host <-> device marshalling and the
tolerance rule).  The expected values always come from the CPU oracle."""
import numpy as np
import torch

# |y - y_ref| <= REL * sum_k |x_k w'_k| + ABS, per element.
REL_TOL = 2e-3
ABS_TOL = 1e-5


def dev():
    return torch.device("cuda:0")


def to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev())


def f16_bits(t):
    """GPU fp16 tensor -> host uint16 bit patterns."""
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def u32_bits(t):
    return t.detach().cpu().contiguous().numpy().view(np.uint32)


def qweight_from_oracle(packed, scales, zeros, group_size, symmetric=False, bits=4):
    """Oracle-produced packed weights as a QuantizedWeight on the GPU."""
    from w4a16_dequant_gemv_amd.api import QuantizedWeight
    n_out, words = packed.shape
    return QuantizedWeight(to_dev(packed.view(np.int32)),
                           to_dev(scales).view(torch.float16),
                           to_dev(zeros).view(torch.float16),
                           n_out, words * (32 // bits), group_size, symmetric, bits)


def assert_within_tolerance(y_gpu, y_ref, a_ref, what=""):
    """y_gpu: GPU fp16 [m][n]; y_ref, a_ref: oracle float64 [m][n]."""
    y = f16_bits(y_gpu).view(np.float16).astype(np.float64)
    assert y.shape == y_ref.shape, (y.shape, y_ref.shape)
    err = np.abs(y - y_ref)
    lim = REL_TOL * a_ref + ABS_TOL
    bad = ~(err <= lim)
    if bad.any():
        i = tuple(np.argwhere(bad)[0])
        raise AssertionError(
            f"{what}: {int(bad.sum())} of {bad.size} outputs outside tolerance; first at {i}: "
            f"y={y[i]!r} ref={y_ref[i]!r} sum|xw'|={a_ref[i]!r}")
    return float((err / np.maximum(a_ref, 1e-30)).max())


def assert_bits_equal(got, want, what):
    got = np.asarray(got)
    want = np.asarray(want)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    neq = got != want
    if neq.any():
        i = tuple(np.argwhere(neq)[0])
        raise AssertionError(f"{what}: {int(neq.sum())} of {neq.size} differ; first at {i}: "
                             f"gpu={hex(int(got[i]))} oracle={hex(int(want[i]))}")


def realign_metadata(qw, align):
    """The same QuantizedWeight with its scale and zero-point arrays copied to
    addresses congruent to `align` modulo 16 (fresh allocations are 256-byte
    aligned; the prefill kernel picks its metadata loads by alignment)."""
    from w4a16_dequant_gemv_amd.api import QuantizedWeight
    off = (align % 16) // 2
    if off == 0:
        return qw

    def moved(t):
        buf = torch.empty(t.numel() + 8, dtype=t.dtype, device=t.device)
        v = buf[off:off + t.numel()].view(t.shape)
        v.copy_(t)
        return v
    return QuantizedWeight(qw.qweight, moved(qw.scales), moved(qw.zeros), qw.n_out, qw.n_in,
                           qw.group_size, qw.symmetric, qw.bits)
