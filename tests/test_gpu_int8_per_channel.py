"""INT8 weights (W8A16) and per-channel groups on the GPU against the CPU oracle:
quantize+pack and dequant bit for bit, the linear layers within the stated
tolerance."""
import numpy as np
import pytest
import torch

import w4a16_dequant_gemv_amd as w4
from gpu_util import assert_bits_equal, assert_within_tolerance, f16_bits, qweight_from_oracle, to_dev, u32_bits
from w4a16_dequant_gemv_amd import synthetic

pytestmark = pytest.mark.gpu


def _quantize_both(orc, w, g, sym, bits):
    qw = w4.quantize_pack(to_dev(w), g, sym, bits=bits)
    torch.cuda.synchronize()
    packed, scales, zeros, _ = orc.quantize_pack(w, g, sym, bits=bits)
    return qw, packed, scales, zeros


def _assert_same(qw, packed, scales, zeros, what):
    assert_bits_equal(u32_bits(qw.qweight), packed, f"{what} packed")
    assert_bits_equal(f16_bits(qw.scales), scales, f"{what} scales")
    assert_bits_equal(f16_bits(qw.zeros), zeros, f"{what} zeros")


@pytest.mark.parametrize("g", [32, 64, 128, 256, None])
@pytest.mark.parametrize("sym", [False, True])
def test_int8_quantize_normal_with_outliers(orc, g, sym):
    w = synthetic.normal_weight(96, 2048, seed=201, std=0.02, n_outlier_cols=4)
    gs = 2048 if g is None else g
    qw, *ref = _quantize_both(orc, w, gs, sym, 8)
    _assert_same(qw, *ref, f"int8 normal g={gs} sym={sym}")


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("shape", [(3, 32), (5, 96), (7, 11008), (16, 4096), (9, 2080), (1, 28672)])
@pytest.mark.parametrize("sym", [False, True])
def test_per_channel_quantize(orc, bits, shape, sym):
    rng = np.random.default_rng(shape[1] + 7 * bits)
    w = (rng.standard_t(3, size=shape) * 0.02).astype(np.float32)
    w[0, :] = np.abs(w[0, :]) + 0.01                       # one all-positive row
    qw, *ref = _quantize_both(orc, w, shape[1], sym, bits)
    _assert_same(qw, *ref, f"per-channel {shape} bits={bits} sym={sym}")


def test_int8_special_rows(orc):
    """Exact ties at s = 1, one-signed rows, constant and tiny rows, per channel and per group."""
    n = 32
    rows = []
    rows.append([-127.0, 128.0, 0.5, 1.5, 2.5, -0.5, -1.5, 3.5, -2.5, 100.5] + [0.0] * 22)
    rows.append(list(np.linspace(0.5, 2.0, n)))
    rows.append(list(np.linspace(-2.0, -0.5, n)))
    for c in (0.75, -0.75, 0.0, -0.0, 3e-9, 2e-8):
        rows.append([c] * n)
    rows.append([1e-10 * i for i in range(n)])
    rows.append([127.0, -126.5, 0.5, 1.5, 2.5, -0.5, -3.5, 5.5] + [0.0] * 24)
    w = np.array(rows, dtype=np.float32)
    for g in (32, n):
        for sym in (False, True):
            qw, *ref = _quantize_both(orc, w, g, sym, 8)
            _assert_same(qw, *ref, f"int8 special g={g} sym={sym}")


@pytest.mark.parametrize("bits,g", [(8, 128), (8, 32), (8, None), (4, None)])
def test_dequant_bit_exact(orc, bits, g):
    w = synthetic.student_t_weight(48, 4096, seed=203, group_size=128, const_frac=0.02, zero_frac=0.01)
    gs = 4096 if g is None else g
    packed, scales, zeros, _ = orc.quantize_pack(w, gs, False, bits=bits)
    qw = qweight_from_oracle(packed, scales, zeros, gs, bits=bits)
    wd = w4.dequant(qw)
    torch.cuda.synchronize()
    want = orc.dequant(packed, scales, zeros, gs, bits=bits)
    assert np.array_equal(wd.cpu().numpy().view(np.uint32), want.view(np.uint32))


@pytest.mark.parametrize("n_out,n_in", [(100, 96), (300, 4096), (64, 11008), (129, 160)])
@pytest.mark.parametrize("m,fn", [(1, "gemv"), (8, "gemv"), (16, "gemv"), (64, "gemm"), (300, "gemm")])
def test_int4_per_channel_linear(orc, n_out, n_in, m, fn):
    w = synthetic.normal_weight(n_out, n_in, seed=n_in + n_out, std=0.02, n_outlier_cols=2)
    packed, scales, zeros, _ = orc.quantize_pack(w, n_in, False)
    qw = qweight_from_oracle(packed, scales, zeros, n_in)
    x = synthetic.activations_f16(m, n_in, seed=m + n_in)
    y = getattr(w4, fn)(to_dev(x), qw)
    y_ref, a_ref = orc.linear_from_packed(x.view(np.uint16), packed, scales, zeros, n_in)
    assert_within_tolerance(y, y_ref, a_ref, f"{fn} per-channel m={m} {n_out}x{n_in}")


Q8_SHAPES = [(100, 96, 32), (128, 256, 128), (300, 4096, None), (64, 11008, None),
             (129, 1088, 64), (256, 2048, 256), (200, 1120, 32), (97, 160, None)]


@pytest.mark.parametrize("n_out,n_in,g", Q8_SHAPES)
@pytest.mark.parametrize("m,fn", [(1, "gemv"), (3, "gemv"), (8, "gemv"), (16, "gemv"),
                                  (64, "gemm"), (300, "gemm")])
@pytest.mark.parametrize("sym", [False, True])
def test_int8_linear(orc, n_out, n_in, g, m, fn, sym):
    gs = n_in if g is None else g
    w = synthetic.student_t_weight(n_out, n_in, seed=5 * n_in + n_out, group_size=32)
    packed, scales, zeros, _ = orc.quantize_pack(w, gs, sym, bits=8)
    qw = qweight_from_oracle(packed, scales, zeros, gs, sym, bits=8)
    x = synthetic.activations_f16(m, n_in, seed=m + 3 * n_in)
    y = getattr(w4, fn)(to_dev(x), qw)
    y_ref, a_ref = orc.linear_from_packed(x.view(np.uint16), packed, scales, zeros, gs, bits=8)
    assert_within_tolerance(y, y_ref, a_ref, f"q8 {fn} m={m} {n_out}x{n_in} g={gs} sym={sym}")


@pytest.mark.parametrize("fn,m", [("gemv", 3), ("gemm", 40)])
@pytest.mark.parametrize("g", [32, None])
def test_int8_one_hot_is_bitwise(orc, fn, m, g):
    """x = e_k selects column k of W': y = fp16(w'[:, k]) exactly, for INT8 codes."""
    n_out, n_in = 160, 1056
    gs = n_in if g is None else g
    w = synthetic.normal_weight(n_out, n_in, seed=207, n_outlier_cols=2)
    packed, scales, zeros, _ = orc.quantize_pack(w, gs, False, bits=8)
    wd = orc.dequant(packed, scales, zeros, gs, bits=8)
    qw = qweight_from_oracle(packed, scales, zeros, gs, bits=8)
    ks = (0, 1, 3, 4, 15, 16, 31, 32, 63, 64, 1023, 1024, 1055)
    x = np.zeros((m, n_in), dtype=np.float16)
    for r, k in enumerate(ks[:m] if m < len(ks) else ks):
        x[r, k] = 1.0
    y = f16_bits(getattr(w4, fn)(to_dev(x), qw))
    for r, k in enumerate(ks[:m] if m < len(ks) else ks):
        assert_bits_equal(y[r], wd[:, k].astype(np.float16).view(np.uint16), f"q8 {fn} one-hot k={k}")
    for r in range(min(m, len(ks)), m):
        assert np.all(y[r] == 0)


def test_int8_rejects_bad_group(orc):
    w = torch.zeros((8, 96), dtype=torch.float32, device="cuda")
    with pytest.raises(w4.W4A16Error):
        w4.quantize_pack(w, 48, bits=8)


@pytest.mark.parametrize("m,n_out,n_in,g", [
    (1, 12301, 4160, None),    # 769 tiles, per-channel, a partial last 128-wide block
    (1, 8200, 16416, None),    # long rows, 513 tiles, a partial last block
    (8, 10250, 4224, 128),     # m > 4, 641 tiles: four tiles per workgroup
    (8, 700, 2080, 32),        # m > 4, two tiles per workgroup, a partial last block
    (1, 130, 2080, 32),        # few tiles, a partial last block
])
def test_int8_paired_loads_ragged(orc, m, n_out, n_in, g):
    """INT8 GEMV shapes on the paired-load rules (two 16-byte halves of a
    block read as whole 128-byte lines of 8 rows), with a partial last tile
    (n_out % 16 != 0); 384 sampled output channels and the last 20 against
    the oracle."""
    gs = n_in if g is None else g
    dev = torch.device("cuda:0")
    w_dev = synthetic.normal_weight_device(n_out, n_in, n_out + 7 * n_in, 0.02, 2, dev)
    x = synthetic.activations_f16(m, n_in, seed=n_in + 5 * m)
    qw = w4.quantize_pack(w_dev, gs, bits=8)
    y = w4.gemv(to_dev(x), qw)
    rows = np.random.default_rng(n_out + 1).choice(n_out, size=min(384, n_out), replace=False)
    rows = np.unique(np.concatenate([rows, np.arange(n_out - 20, n_out)]))
    w_rows = w_dev[torch.from_numpy(rows).to(dev)].cpu().numpy()
    del w_dev
    packed, scales, zeros, _ = orc.quantize_pack(w_rows, gs, False, bits=8)
    y_ref, a_ref = orc.linear_from_packed(x.view(np.uint16), packed, scales, zeros, gs, bits=8)
    assert_within_tolerance(y[:, torch.from_numpy(rows).to(dev)], y_ref, a_ref,
                            f"q8 paired {m}x{n_out}x{n_in} g={gs}")
