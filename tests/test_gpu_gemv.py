"""Decode GEMV (m <= 16) against the oracle's binary64 product on the
oracle-dequantized weights, within |y - y_ref| <= 2e-3 sum|x w'| + 1e-5."""
import numpy as np
import pytest
import torch

import w4a16_dequant_gemv_amd as w4
from gpu_util import (assert_bits_equal, assert_within_tolerance, f16_bits,
                      qweight_from_oracle, to_dev)
from w4a16_dequant_gemv_amd import synthetic

pytestmark = pytest.mark.gpu


def _check(orc, w, x, g, sym=False, what=""):
    """Quantize on both sides, run the GPU GEMV, compare to the oracle."""
    packed, scales, zeros, _ = orc.quantize_pack(w, g, sym)
    qw = w4.quantize_pack(to_dev(w), g, sym)
    y = w4.gemv(to_dev(x), qw)
    torch.cuda.synchronize()
    y_ref, a_ref = orc.linear_from_packed(x.view(np.uint16), packed, scales, zeros, g)
    return assert_within_tolerance(y, y_ref, a_ref, what)


SHAPES = [(1, 32, 32), (16, 128, 128), (17, 96, 32), (100, 4096, 128), (64, 11008, 128),
          (33, 256, 256), (48, 192, 64), (256, 8192, 128), (40, 4128, 32), (7, 1024, 64)]


@pytest.mark.parametrize("m", [1, 2, 3, 4, 5, 8, 15, 16])
@pytest.mark.parametrize("n_out,n_in,g", SHAPES)
def test_gemv_shapes(orc, m, n_out, n_in, g):
    w = synthetic.normal_weight(n_out, n_in, seed=n_out * 7 + n_in, std=0.02,
                                n_outlier_cols=synthetic.n_outliers(n_in))
    x = synthetic.activations_f16(m, n_in, seed=m * 13 + n_in)
    _check(orc, w, x, g, what=f"m={m} {n_out}x{n_in} g={g}")


@pytest.mark.parametrize("g,sym", [(32, False), (32, True), (128, True), (256, False)])
def test_gemv_modes(orc, g, sym):
    w = synthetic.student_t_weight(200, 2048, seed=201, group_size=g)
    x = synthetic.activations_f16(4, 2048, seed=202)
    _check(orc, w, x, g, sym, f"student-t g={g} sym={sym}")


def test_gemv_one_hot_is_bitwise(orc):
    """x = e_k selects column k of W': y = fp16(w'[:, k]) exactly."""
    n_out, n_in, g = 96, 1024, 128
    w = synthetic.normal_weight(n_out, n_in, seed=203, n_outlier_cols=2)
    packed, scales, zeros, _ = orc.quantize_pack(w, g)
    wd = orc.dequant(packed, scales, zeros, g)
    qw = qweight_from_oracle(packed, scales, zeros, g)
    for k in (0, 1, 7, 8, 31, 32, 127, 128, 511, 1023):
        x = np.zeros((3, n_in), dtype=np.float16)
        x[0, k] = 1.0
        x[2, (k + 5) % n_in] = 1.0
        y = f16_bits(w4.gemv(to_dev(x), qw))
        assert_bits_equal(y[0], wd[:, k].astype(np.float16).view(np.uint16), f"one-hot k={k}")
        assert np.all(y[1] == 0)
        assert_bits_equal(y[2], wd[:, (k + 5) % n_in].astype(np.float16).view(np.uint16),
                          f"one-hot row 2 k={k}")


def test_gemv_zero_weights_give_zero(orc):
    w = np.zeros((64, 512), dtype=np.float32)
    x = synthetic.activations_f16(2, 512, seed=204)
    qw = w4.quantize_pack(to_dev(w), 128)
    y = w4.gemv(to_dev(x), qw).float().cpu().numpy()
    assert np.all(y == 0)


def test_gemv_deterministic():
    w = to_dev(synthetic.normal_weight(4096, 4096, seed=205))
    x = to_dev(synthetic.activations_f16(8, 4096, seed=206))
    qw = w4.quantize_pack(w, 128)
    a = w4.gemv(x, qw)
    b = w4.gemv(x, qw)
    assert torch.equal(a, b)


def test_gemv_empty_batch():
    qw = w4.quantize_pack(to_dev(np.ones((16, 128), np.float32)), 128)
    y = w4.gemv(torch.zeros((0, 128), dtype=torch.float16, device="cuda"), qw)
    assert y.shape == (0, 16)


def test_gemv_rejects_17_rows():
    qw = w4.quantize_pack(to_dev(np.ones((16, 128), np.float32)), 128)
    with pytest.raises(w4.W4A16Error):
        w4.gemv(torch.zeros((17, 128), dtype=torch.float16, device="cuda"), qw)


# --------------------------------------------------------------------------
# Full-size workloads, in the launch configuration the benchmark uses.
# --------------------------------------------------------------------------
def test_gemv_single_linear_4096(orc):
    """W[4096, 4096] ~ N(0, 0.02), 8 outlier columns, g=128, x[1, 4096]: every output."""
    w = synthetic.normal_weight(4096, 4096, seed=1, std=0.02, n_outlier_cols=8)
    x = synthetic.activations_f16(1, 4096, seed=101)
    _check(orc, w, x, 128, what="4096x4096 m=1")


def test_gemv_llama7b_layer(orc):
    """All seven linears of one 7B-shaped layer at m=1: every output."""
    x_all = {}
    for i, lin in enumerate(synthetic.LLAMA7B_LINEARS):
        w = synthetic.normal_weight(lin.n_out, lin.n_in, seed=synthetic.llama7b_seed(0, i),
                                    std=0.02, n_outlier_cols=synthetic.n_outliers(lin.n_in))
        if lin.n_in not in x_all:
            x_all[lin.n_in] = synthetic.activations_f16(1, lin.n_in, seed=2100 + lin.n_in)
        _check(orc, w, x_all[lin.n_in], 128, what=f"7B {lin.name}")


def test_gemv_llama70b_m8_sampled_rows(orc):
    """70B-shaped linears at m=8 (layer 0), weights drawn on the GPU; 384
    sampled output channels per linear are checked against the oracle."""
    dev = torch.device("cuda:0")
    rng = np.random.default_rng(207)
    for i, lin in enumerate(synthetic.LLAMA70B_LINEARS):
        w_dev = synthetic.normal_weight_device(lin.n_out, lin.n_in, synthetic.llama70b_seed(0, i),
                                               0.015, 0, dev)
        x = synthetic.activations_f16(8, lin.n_in, seed=3100 + i)
        qw = w4.quantize_pack(w_dev, 128)
        y = w4.gemv(to_dev(x), qw)
        rows = np.sort(rng.choice(lin.n_out, size=min(384, lin.n_out), replace=False))
        w_rows = w_dev[torch.from_numpy(rows).to(dev)].cpu().numpy()
        del w_dev
        packed, scales, zeros, _ = orc.quantize_pack(w_rows, 128)
        y_ref, a_ref = orc.linear_from_packed(x.view(np.uint16), packed, scales, zeros, 128)
        y_rows = y[:, torch.from_numpy(rows).to(dev)]
        assert_within_tolerance(y_rows, y_ref, a_ref, f"70B {lin.name} m=8")


@pytest.mark.parametrize("m,n_out,n_in,g", [
    (1, 12301, 8320, 128),     # rows of 8192+ codes, 769 tiles: two tiles per workgroup
    (1, 8200, 16512, 128),     # long rows, 513 tiles: one tile per workgroup
    (1, 8200, 16416, 32),      # the same without the scale fold; a partial last block
    (3, 10250, 4224, 128),     # m > 1, 641 tiles: four tiles per workgroup
])
def test_gemv_paired_loads_ragged(orc, m, n_out, n_in, g):
    """The dispatch rules that read weights as whole 128-byte lines of 8 rows,
    on shapes with a partial last tile (n_out % 16 != 0) and an odd number of
    128-wide blocks (the last pair's second block lies past the end) or a
    partial last block; 384 sampled output channels and the last 20 against
    the oracle."""
    dev = torch.device("cuda:0")
    w_dev = synthetic.normal_weight_device(n_out, n_in, n_out + n_in, 0.02, 2, dev)
    x = synthetic.activations_f16(m, n_in, seed=n_in + m)
    qw = w4.quantize_pack(w_dev, g)
    y = w4.gemv(to_dev(x), qw)
    rows = np.random.default_rng(n_out).choice(n_out, size=384, replace=False)
    rows = np.unique(np.concatenate([rows, np.arange(n_out - 20, n_out)]))
    w_rows = w_dev[torch.from_numpy(rows).to(dev)].cpu().numpy()
    del w_dev
    packed, scales, zeros, _ = orc.quantize_pack(w_rows, g)
    y_ref, a_ref = orc.linear_from_packed(x.view(np.uint16), packed, scales, zeros, g)
    assert_within_tolerance(y[:, torch.from_numpy(rows).to(dev)], y_ref, a_ref, f"paired {m}x{n_out}x{n_in} g={g}")


@pytest.fixture(scope="module")
def stress_weights():
    """8192x28672 Student-t weights per group size (constant groups are placed
    on whole groups of that size); drawn once per module."""
    cache = {}

    def get(g):
        if g not in cache:
            cache[g] = synthetic.student_t_weight(8192, 28672, seed=5, group_size=g)
        return cache[g]
    return get


@pytest.mark.parametrize("g,sym", [(128, False), (32, False), (128, True), (32, True)])
def test_gemv_stress_8192x28672(orc, stress_weights, g, sym):
    """Heavy-tailed 8192x28672 weights with constant groups, m=1; the
    quantization is compared bit for bit on sampled rows and y on every
    output against the oracle's product for those rows."""
    w = stress_weights(g)
    x = synthetic.activations_f16(1, 28672, seed=5100)
    qw = w4.quantize_pack(to_dev(w), g, sym)
    y = w4.gemv(to_dev(x), qw)
    rows = np.sort(np.random.default_rng(208).choice(8192, size=512, replace=False))
    packed, scales, zeros, _ = orc.quantize_pack(w[rows], g, sym)
    idx = torch.from_numpy(rows).to(y.device)
    assert_bits_equal(qw.qweight[idx].cpu().numpy().view(np.uint32), packed, "stress packed")
    assert_bits_equal(f16_bits(qw.scales[idx]), scales, "stress scales")
    y_ref, a_ref = orc.linear_from_packed(x.view(np.uint16), packed, scales, zeros, g)
    assert_within_tolerance(y[:, idx], y_ref, a_ref, f"stress g={g} sym={sym}")
