"""GPU quantize+pack and dequant against the CPU oracle, bit for bit."""
import numpy as np
import pytest
import torch

import w4a16_dequant_gemv_amd as w4
from gpu_util import assert_bits_equal, f16_bits, to_dev, u32_bits
from w4a16_dequant_gemv_amd import synthetic

pytestmark = pytest.mark.gpu

MODES = [(g, sym) for g in (32, 64, 128, 256) for sym in (False, True)]


def _quantize_both(orc, w, g, sym):
    qw = w4.quantize_pack(to_dev(w), g, sym)
    torch.cuda.synchronize()
    packed, scales, zeros, _ = orc.quantize_pack(w, g, sym)
    return qw, packed, scales, zeros


def _assert_same(qw, packed, scales, zeros, what):
    assert_bits_equal(u32_bits(qw.qweight), packed, f"{what} packed")
    assert_bits_equal(f16_bits(qw.scales), scales, f"{what} scales")
    assert_bits_equal(f16_bits(qw.zeros), zeros, f"{what} zeros")


@pytest.mark.parametrize("g,sym", MODES)
def test_quantize_normal_with_outliers(orc, g, sym):
    w = synthetic.normal_weight(96, 2048, seed=101, std=0.02, n_outlier_cols=4)
    qw, *ref = _quantize_both(orc, w, g, sym)
    _assert_same(qw, *ref, f"normal g={g} sym={sym}")


@pytest.mark.parametrize("g,sym", MODES)
def test_quantize_student_t_with_constant_groups(orc, g, sym):
    w = synthetic.student_t_weight(64, 4096, seed=102, group_size=g, const_frac=0.05,
                                   zero_frac=0.02)
    qw, *ref = _quantize_both(orc, w, g, sym)
    _assert_same(qw, *ref, f"student-t g={g} sym={sym}")


@pytest.mark.parametrize("shape,g", [((1, 32), 32), ((5, 32), 32), ((3, 96), 32),
                                     ((7, 11008), 128), ((1, 256), 256), ((33, 192), 64),
                                     ((2, 4096), 128)])
@pytest.mark.parametrize("sym", [False, True])
def test_quantize_edge_shapes(orc, shape, g, sym):
    rng = np.random.default_rng(hash(shape) % 2**32)
    w = (rng.standard_normal(shape) * 0.3).astype(np.float32)
    qw, *ref = _quantize_both(orc, w, g, sym)
    _assert_same(qw, *ref, f"{shape} g={g} sym={sym}")


def test_quantize_special_groups(orc):
    """Ties, one-signed groups, constant groups, tiny ranges, subnormal inputs."""
    g = 32
    rows = []
    rows.append([-7.0, 8.0, 0.5, 1.5, 2.5, -0.5, -1.5, 3.5] + [0.0] * 24)      # exact ties
    rows.append(list(np.linspace(0.5, 2.0, g)))                                 # all positive
    rows.append(list(np.linspace(-2.0, -0.5, g)))                               # all negative
    for c in (0.75, -0.75, 0.0, -0.0, 3e-9, 2e-8, 1e-30):
        rows.append([c] * g)                                                    # constant
    rows.append([1e-9 * i for i in range(g)])                                   # range < 15e-8
    rows.append([1e-40 * (i - 16) for i in range(g)])                           # fp32 subnormals
    rows.append([7.0, -6.5, 0.5, 1.5, 2.5, -0.5, -3.5, 5.5] + [0.0] * 24)      # symmetric ties
    w = np.array(rows, dtype=np.float32)
    for sym in (False, True):
        qw, *ref = _quantize_both(orc, w, g, sym)
        _assert_same(qw, *ref, f"special sym={sym}")


@pytest.mark.parametrize("g,sym", [(128, False), (128, True), (32, False), (32, True)])
def test_quantize_config1_full(orc, g, sym):
    """W[4096, 4096] ~ N(0, 0.02) with 8 outlier columns, every element."""
    w = synthetic.normal_weight(4096, 4096, seed=1, std=0.02, n_outlier_cols=8)
    qw, *ref = _quantize_both(orc, w, g, sym)
    _assert_same(qw, *ref, f"4096x4096 g={g} sym={sym}")


def test_dequant_bit_exact(orc):
    rng = np.random.default_rng(103)
    for g in (32, 64, 128, 256):
        n_out, n_in = 40, 1024
        packed = rng.integers(0, 1 << 32, size=(n_out, n_in // 8), dtype=np.uint64).astype(np.uint32)
        s = rng.uniform(0, 0.1, size=(n_out, n_in // g)).astype(np.float16)
        s[0, 0] = 0.0
        s[1, 0] = np.float16(6e-8)
        z = rng.integers(0, 16, size=(n_out, n_in // g)).astype(np.float16)
        qw = w4.QuantizedWeight(to_dev(packed.view(np.int32)), to_dev(s), to_dev(z),
                                n_out, n_in, g)
        got = w4.dequant(qw).cpu().numpy()
        want = orc.dequant(packed, s.view(np.uint16), z.view(np.uint16), g)
        assert_bits_equal(got.view(np.uint32), want.view(np.uint32), f"dequant g={g}")


def test_quantize_dequant_roundtrip_matches_oracle(orc):
    w = synthetic.student_t_weight(128, 4096, seed=104, group_size=128)
    for sym in (False, True):
        qw = w4.quantize_pack(to_dev(w), 128, sym)
        got = w4.dequant(qw).cpu().numpy()
        packed, scales, zeros, _ = orc.quantize_pack(w, 128, sym)
        want = orc.dequant(packed, scales, zeros, 128)
        assert_bits_equal(got.view(np.uint32), want.view(np.uint32), f"round trip sym={sym}")


def test_quantize_is_deterministic():
    w = to_dev(synthetic.normal_weight(256, 4096, seed=105))
    a = w4.quantize_pack(w, 128)
    b = w4.quantize_pack(w, 128)
    assert torch.equal(a.qweight, b.qweight) and torch.equal(a.scales, b.scales)
