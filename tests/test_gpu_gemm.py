"""Prefill GEMM against the oracle's binary64 product on the oracle-dequantized
weights, within |y - y_ref| <= 2e-3 sum|x w'| + 1e-5."""
import numpy as np
import pytest
import torch

import w4a16_dequant_gemv_amd as w4
from gpu_util import assert_bits_equal, assert_within_tolerance, f16_bits, qweight_from_oracle, to_dev
from w4a16_dequant_gemv_amd import synthetic

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("m", [1, 17, 64, 127, 128, 129, 300])
@pytest.mark.parametrize("n_out,n_in,g", [(1, 32, 32), (100, 96, 32), (128, 256, 128),
                                          (300, 4096, 128), (129, 1088, 64), (64, 512, 256),
                                          (200, 1120, 32), (64, 160, 32), (48, 192, 64)])
def test_gemm_shapes(orc, m, n_out, n_in, g):
    w = synthetic.normal_weight(n_out, n_in, seed=n_out + 3 * n_in, std=0.02,
                                n_outlier_cols=synthetic.n_outliers(n_in))
    x = synthetic.activations_f16(m, n_in, seed=m + 5 * n_in)
    packed, scales, zeros, _ = orc.quantize_pack(w, g)
    qw = w4.quantize_pack(to_dev(w), g)
    y = w4.gemm(to_dev(x), qw)
    torch.cuda.synchronize()
    y_ref, a_ref = orc.linear_from_packed(x.view(np.uint16), packed, scales, zeros, g)
    assert_within_tolerance(y, y_ref, a_ref, f"m={m} {n_out}x{n_in} g={g}")


def test_gemm_matches_gemv_domain(orc):
    """m <= 16 through the GEMM entry point also meets the bound."""
    w = synthetic.student_t_weight(256, 2048, seed=301, group_size=32)
    x = synthetic.activations_f16(16, 2048, seed=302)
    for sym in (False, True):
        packed, scales, zeros, _ = orc.quantize_pack(w, 32, sym)
        qw = qweight_from_oracle(packed, scales, zeros, 32, sym)
        y_ref, a_ref = orc.linear_from_packed(x.view(np.uint16), packed, scales, zeros, 32)
        assert_within_tolerance(w4.gemm(to_dev(x), qw), y_ref, a_ref, f"gemm m=16 sym={sym}")
        assert_within_tolerance(w4.linear(to_dev(x), qw), y_ref, a_ref, f"linear m=16 sym={sym}")


def test_gemm_one_hot_is_bitwise(orc):
    n_out, n_in, g = 160, 512, 128
    w = synthetic.normal_weight(n_out, n_in, seed=303)
    packed, scales, zeros, _ = orc.quantize_pack(w, g)
    wd = orc.dequant(packed, scales, zeros, g)
    qw = qweight_from_oracle(packed, scales, zeros, g)
    m = 130
    x = np.zeros((m, n_in), dtype=np.float16)
    ks = [(i * 37) % n_in for i in range(m)]
    for i, k in enumerate(ks):
        x[i, k] = 1.0
    y = f16_bits(w4.gemm(to_dev(x), qw))
    for i, k in enumerate(ks):
        assert_bits_equal(y[i], wd[:, k].astype(np.float16).view(np.uint16), f"row {i} k={k}")


def test_gemm_deterministic():
    w = to_dev(synthetic.normal_weight(512, 4096, seed=304))
    x = to_dev(synthetic.activations_f16(256, 4096, seed=305))
    qw = w4.quantize_pack(w, 128)
    assert torch.equal(w4.gemm(x, qw), w4.gemm(x, qw))


@pytest.mark.parametrize("idx", range(len(synthetic.PREFILL_LINEARS)))
def test_gemm_prefill_2048_sampled_rows(orc, idx):
    """M=2048 prefill on the 7B shapes: 48 sampled rows of y, every column."""
    lin = synthetic.PREFILL_LINEARS[idx]
    w = synthetic.normal_weight(lin.n_out, lin.n_in, seed=4000 + idx, std=0.02,
                                n_outlier_cols=synthetic.n_outliers(lin.n_in))
    x = synthetic.activations_f16(synthetic.PREFILL_M, lin.n_in, seed=4100 + idx)
    qw = w4.quantize_pack(to_dev(w), 128)
    y = w4.gemm(to_dev(x), qw)
    rows = np.sort(np.random.default_rng(306 + idx).choice(synthetic.PREFILL_M, 48, replace=False))
    rows[0], rows[-1] = 0, synthetic.PREFILL_M - 1
    packed, scales, zeros, _ = orc.quantize_pack(w, 128)
    y_ref, a_ref = orc.linear_from_packed(x[rows].view(np.uint16), packed, scales, zeros, 128)
    assert_within_tolerance(y[torch.from_numpy(rows).to(y.device)], y_ref, a_ref,
                            f"prefill {lin.n_out}x{lin.n_in}")


def _with_meta_offset(qw, offset):
    """The same weights with scales and zeros copied `offset` halves into
    fresh buffers (offset 1: only 2-byte aligned, 2: 4-byte aligned)."""
    from w4a16_dequant_gemv_amd.api import QuantizedWeight

    def moved(t):
        buf = torch.zeros(t.numel() + 8, dtype=t.dtype, device=t.device)
        view = buf[offset:offset + t.numel()].view(t.shape)
        view.copy_(t)
        return view
    return QuantizedWeight(qw.qweight, moved(qw.scales), moved(qw.zeros), qw.n_out, qw.n_in, qw.group_size,
                           qw.symmetric, qw.bits)


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("n_out,n_in,g", [(96, 1024, 64), (80, 2048, 256), (72, 4608, 256), (64, 640, 64),
                                          (130, 4096, 128), (40, 2816, 128), (33, 1088, 64)])
def test_gemm_scale_runs(orc, bits, n_out, n_in, g):
    """Groups of 64..256: the producers read runs of 8 (16-byte aligned
    metadata, groups per row a multiple of 8) or 2 (4-byte aligned, even)
    groups' scales and zero-points at once, else one per step.  Every form
    gives the same bits, within tolerance of the oracle."""
    w = synthetic.normal_weight(n_out, n_in, seed=7 * n_out + n_in, std=0.02,
                                n_outlier_cols=synthetic.n_outliers(n_in))
    x = synthetic.activations_f16(300, n_in, seed=11 + n_in)
    packed, scales, zeros, _ = orc.quantize_pack(w, g, bits=bits)
    qw = qweight_from_oracle(packed, scales, zeros, g, bits=bits)
    xd = to_dev(x)
    ys = [w4.gemm(xd, _with_meta_offset(qw, off)) for off in (0, 1, 2)]
    torch.cuda.synchronize()
    y_ref, a_ref = orc.linear_from_packed(x.view(np.uint16), packed, scales, zeros, g, bits=bits)
    assert_within_tolerance(ys[0], y_ref, a_ref, f"q{bits} gemm {n_out}x{n_in} g={g}")
    for off, y in zip((1, 2), ys[1:]):
        assert_bits_equal(f16_bits(y), f16_bits(ys[0]), f"q{bits} gemm {n_out}x{n_in} g={g} metadata offset {off}")
