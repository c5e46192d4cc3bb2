"""W8A8 with SmoothQuant on the GPU against the CPU oracle, bit for bit:
calibration maxima, smoothing factors, per-channel INT8 weights, per-token
INT8 activations and the int8 product (y itself is bit-exact: the integer
sums are exact and the epilogue is a fixed binary32 sequence)."""
import numpy as np
import pytest
import torch

from gpu_util import to_dev
from w4a16_dequant_gemv_amd import synthetic, w8a8

pytestmark = pytest.mark.gpu


def _act(m, k, seed, outliers=3):
    """fp16 activations ~ N(0, 1) with a few x60 outlier channels."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((m, k)).astype(np.float32)
    x[:, rng.choice(k, min(outliers, k), replace=False)] *= 60.0
    return x.astype(np.float16)


def _eq(got, want, what):
    got = got.cpu().numpy()
    assert got.shape == want.shape, (what, got.shape, want.shape)
    if got.dtype in (np.float32, np.float16):
        got = got.view(np.uint32 if got.dtype == np.float32 else np.uint16)
        want = want.view(got.dtype)
    bad = np.argwhere(got != want)
    assert bad.size == 0, f"{what}: {len(bad)} mismatches, first at {bad[:3].tolist()}"


def test_absmax_accumulates(orc):
    x1, x2 = _act(300, 4096, 1), _act(77, 4096, 2)
    w = synthetic.normal_weight(513, 4096, seed=3, n_outlier_cols=4)
    a = torch.zeros(4096, dtype=torch.float32, device="cuda")
    w8a8.absmax_update(to_dev(x1), a)
    w8a8.absmax_update(to_dev(x2), a)
    wm = torch.zeros(4096, dtype=torch.float32, device="cuda")
    w8a8.absmax_update(to_dev(w), wm)
    torch.cuda.synchronize()
    want = np.maximum(orc.col_absmax_f16(x1.view(np.uint16)), orc.col_absmax_f16(x2.view(np.uint16)))
    _eq(a, want, "activation maxima")
    _eq(wm, orc.col_absmax_f32(w), "weight maxima")


@pytest.mark.parametrize("alpha", [0.5, 0.0, 1.0, 0.75])
def test_smooth_factors(orc, alpha):
    rng = np.random.default_rng(4)
    a = np.abs(rng.standard_normal(4096) * 5).astype(np.float32)
    wm = np.abs(rng.standard_normal(4096) * 0.05).astype(np.float32)
    a[:5] = 0.0
    wm[5:10] = 0.0
    s = w8a8.smooth_factors(to_dev(a), to_dev(wm), alpha)
    torch.cuda.synchronize()
    want = orc.smooth_factors(a, wm, alpha)
    if alpha == 0.5:
        _eq(s, want, "factors")
    else:
        # two powf calls per factor, each within about 2 ulp of the true power
        # on either side (device and host libm), and one division: the two
        # results stay within 2 * (2 + 2) + 1 < 10 ulp of each other
        got = s.cpu().numpy()
        ulp = np.abs(np.spacing(want))
        assert (np.abs(got - want) <= 10 * ulp).all(), np.max(np.abs(got - want) / ulp)


@pytest.mark.parametrize("smooth", [False, True])
@pytest.mark.parametrize("n_out,k", [(1, 32), (37, 96), (300, 4096), (64, 11008), (17, 28672), (5, 32768)])
def test_quantize_weight(orc, smooth, n_out, k):
    w = synthetic.normal_weight(n_out, k, seed=n_out + k, n_outlier_cols=2)
    s = (np.abs(np.random.default_rng(k).standard_normal(k)) + 0.1).astype(np.float32) if smooth else None
    qw, sw = w8a8.quantize_weight(to_dev(w), None if s is None else to_dev(s))
    torch.cuda.synchronize()
    q_ref, s_ref = orc.w8a8_quant_weight(w, s)
    _eq(qw, q_ref, f"codes {n_out}x{k}")
    _eq(sw, s_ref, f"scales {n_out}x{k}")


@pytest.mark.parametrize("smooth", [False, True])
@pytest.mark.parametrize("m,k", [(1, 32), (5, 4096), (300, 11008), (64, 28672), (2048, 4096), (3, 32768), (9, 160)])
def test_quantize_act(orc, smooth, m, k):
    x = _act(m, k, seed=m * 3 + k)
    if m > 3:
        x[1] = 0.0                                   # an all-zero token
        x[2, 0] = 65504.0
    s = (np.abs(np.random.default_rng(k + 1).standard_normal(k)) + 0.05).astype(np.float32) if smooth else None
    qx, sx = w8a8.quantize_act(to_dev(x), None if s is None else to_dev(s))
    torch.cuda.synchronize()
    q_ref, s_ref = orc.w8a8_quant_act(x.view(np.uint16), s)
    _eq(qx, q_ref, f"codes {m}x{k}")
    _eq(sx, s_ref, f"scales {m}x{k}")


@pytest.mark.parametrize("m,n,k", [(1, 1, 32), (300, 200, 1120), (257, 129, 4096), (64, 160, 96),
                                   (33, 4096, 224), (130, 256, 64), (512, 384, 11008), (256, 128, 128),
                                   (7, 1000, 28672)])
def test_gemm_bit_exact(orc, m, n, k):
    rng = np.random.default_rng(m + n + k)
    qx = rng.integers(-128, 128, size=(m, k)).astype(np.int8)
    qw = rng.integers(-128, 128, size=(n, k)).astype(np.int8)
    sx = (rng.uniform(0.5, 2, m) * 1e-2).astype(np.float32)
    sw = (rng.uniform(0.5, 2, n) * 1e-3).astype(np.float32)
    y = w8a8.gemm(to_dev(qx), to_dev(sx), to_dev(qw), to_dev(sw))
    torch.cuda.synchronize()
    y_ref, _ = orc.w8a8_gemm(qx, sx, qw, sw)
    _eq(y, y_ref, f"y {m}x{n}x{k}")


@pytest.mark.parametrize("idx", range(len(synthetic.PREFILL_LINEARS)))
def test_prefill_2048_sampled_rows(orc, idx):
    """M = 2048 prefill on the 7B shapes through the whole smoothed path
    (calibration on other tokens, factors, weight and activation codes, the
    product); 48 sampled rows of y against the oracle, bit for bit."""
    lin = synthetic.PREFILL_LINEARS[idx]
    dev = torch.device("cuda")
    w = synthetic.normal_weight_device(lin.n_out, lin.n_in, 7000 + idx, 0.02, synthetic.n_outliers(lin.n_in), dev)
    calib = synthetic.activations_f16_device(512, lin.n_in, 7100 + idx, dev)
    x = synthetic.activations_f16_device(synthetic.PREFILL_M, lin.n_in, 7200 + idx, dev)
    act_max = torch.zeros(lin.n_in, dtype=torch.float32, device=dev)
    w8a8.absmax_update(calib, act_max)
    layer = w8a8.W8A8Linear.from_float(w, act_max)
    y = layer(x)
    torch.cuda.synchronize()
    rows = np.sort(np.random.default_rng(7300 + idx).choice(synthetic.PREFILL_M, 48, replace=False))
    rows[0], rows[-1] = 0, synthetic.PREFILL_M - 1
    s = layer.s.cpu().numpy()
    a_ref = orc.col_absmax_f16(calib.cpu().numpy().view(np.uint16))
    _eq(act_max, a_ref, "calibration maxima")
    w_h = w.cpu().numpy()
    s_ref = orc.smooth_factors(a_ref, orc.col_absmax_f32(w_h), 0.5)
    _eq(layer.s, s_ref, "factors")
    qw_ref, sw_ref = orc.w8a8_quant_weight(w_h, s_ref)
    _eq(layer.qw, qw_ref, "weight codes")
    _eq(layer.sw, sw_ref, "weight scales")
    xr = x[torch.from_numpy(rows).to(dev)].cpu().numpy().view(np.uint16)
    qx_ref, sx_ref = orc.w8a8_quant_act(xr, s)
    y_ref, _ = orc.w8a8_gemm(qx_ref, sx_ref, qw_ref, sw_ref)
    _eq(y[torch.from_numpy(rows).to(dev)], y_ref, f"y {lin.n_out}x{lin.n_in}")


def test_smoothing_reduces_error_on_outlier_activations():
    """On activations with x60 outlier channels the smoothed W8A8 product is
    closer to the fp32 product than the unsmoothed one."""
    dev = torch.device("cuda")
    w = synthetic.normal_weight_device(1024, 4096, 7400, 0.02, 0, dev)
    x = to_dev(_act(256, 4096, 7401, outliers=8))
    ref = x.float() @ w.t()
    act_max = torch.zeros(4096, dtype=torch.float32, device=dev)
    w8a8.absmax_update(x, act_max)
    smoothed = w8a8.W8A8Linear.from_float(w, act_max)(x).float()
    qw, sw = w8a8.quantize_weight(w)
    qx, sx = w8a8.quantize_act(x)
    plain = w8a8.gemm(qx, sx, qw, sw).float()
    e_s = (smoothed - ref).abs().mean().item()
    e_p = (plain - ref).abs().mean().item()
    assert e_s < 0.5 * e_p, (e_s, e_p)
