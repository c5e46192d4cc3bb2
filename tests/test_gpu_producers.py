"""GPTQ and AWQ on the GPU against the CPU oracle, bit for bit: the factor U,
the column loop (fed the oracle's own U, and end to end), AWQ's errors,
winning index, scales and packed weights."""
import numpy as np
import pytest
import torch

from gpu_util import f16_bits, to_dev, u32_bits
from w4a16_dequant_gemv_amd import producers, synthetic

pytestmark = pytest.mark.gpu


def _calib(t, n, seed, outliers=3):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((t, n)).astype(np.float32)
    x[:, rng.choice(n, outliers, replace=False)] *= 8.0
    return x.astype(np.float16)


def _eq(got, want, what):
    got = got.cpu().numpy() if isinstance(got, torch.Tensor) else got
    assert got.shape == want.shape, (what, got.shape, want.shape)
    if got.dtype in (np.float32, np.float64):
        got = got.view(np.uint32 if got.dtype == np.float32 else np.uint64)
        want = want.view(got.dtype)
    bad = np.argwhere(got != want)
    assert bad.size == 0, f"{what}: {len(bad)} mismatches of {got.size}, first at {bad[:3].tolist()}"


@pytest.mark.parametrize("t,n", [(100, 64), (512, 96), (300, 256), (512, 1024)])
def test_gptq_factor_bit_exact(orc, t, n):
    x = _calib(t, n, seed=t + n)
    u = producers.gptq_factor(to_dev(x))
    torch.cuda.synchronize()
    h = orc.gptq_damp(orc.gptq_hessian(x.view(np.uint16)), 0.01)
    want = orc.gptq_hinv_chol(h).astype(np.float32)
    _eq(u, want, f"U t={t} n={n}")


CASES = [  # (n_out, n, group, bits, symmetric)
    (5, 256, 32, 4, False), (37, 1024, 128, 4, False), (64, 512, 128, 4, True), (7, 1088, 64, 4, False),
    (9, 96, 32, 4, False), (12, 384, 384, 4, False), (8, 1024, 256, 4, False), (16, 512, 128, 8, False),
    (10, 640, 64, 8, True), (70, 256, 128, 4, False),
]


@pytest.mark.parametrize("n_out,n,g,bits,sym", CASES)
def test_gptq_loop_with_oracle_factor(orc, n_out, n, g, bits, sym):
    w = synthetic.normal_weight(n_out, n, seed=n_out * 7 + n, n_outlier_cols=2)
    x = _calib(256, n, seed=n + 1)
    u = orc.gptq_hinv_chol(orc.gptq_damp(orc.gptq_hessian(x.view(np.uint16)), 0.01)).astype(np.float32)
    qw = producers.gptq_quantize(to_dev(w), to_dev(u), g, bits, sym)
    torch.cuda.synchronize()
    packed, scales, zeros, _ = orc.gptq_quantize(w, u, g, bits, sym)
    _eq(u32_bits(qw.qweight), packed, "codes")
    _eq(f16_bits(qw.scales), scales, "scales")
    _eq(f16_bits(qw.zeros), zeros, "zeros")


@pytest.mark.parametrize("n_out,n,g", [(48, 512, 128), (33, 1024, 32)])
def test_gptq_end_to_end(orc, n_out, n, g):
    w = synthetic.normal_weight(n_out, n, seed=n_out + 3 * n, n_outlier_cols=2)
    x = _calib(384, n, seed=5 * n)
    qw = producers.gptq(to_dev(w), to_dev(x), g)
    torch.cuda.synchronize()
    packed, scales, zeros = orc.gptq(w, x.view(np.uint16), g)
    _eq(u32_bits(qw.qweight), packed, "codes")
    _eq(f16_bits(qw.scales), scales, "scales")
    _eq(f16_bits(qw.zeros), zeros, "zeros")


def test_gptq_beats_rounding_on_the_gpu(orc):
    """The GPU result lowers the output error against plain rounding."""
    import w4a16_dequant_gemv_amd as w4
    n_out, n = 256, 1024
    w = synthetic.normal_weight(n_out, n, seed=17, n_outlier_cols=2)
    x = _calib(512, n, seed=18)
    g = producers.gptq(to_dev(w), to_dev(x), 128)
    r = w4.quantize_pack(to_dev(w), 128)
    xd = to_dev(x).double()
    wd = to_dev(w).double()
    e_g = ((xd @ (wd - w4.dequant(g).double()).t()) ** 2).sum().item()
    e_r = ((xd @ (wd - w4.dequant(r).double()).t()) ** 2).sum().item()
    assert e_g < e_r, (e_g, e_r)


@pytest.mark.parametrize("n_out,n,t,g,bits,sym,grid", [(16, 256, 64, 128, 4, False, 20), (40, 512, 100, 64, 4, False, 10),
                                                      (24, 256, 50, 128, 8, True, 5), (10, 384, 33, 384, 4, False, 4)])
def test_awq_bit_exact(orc, n_out, n, t, g, bits, sym, grid):
    w = synthetic.normal_weight(n_out, n, seed=n_out + n, n_outlier_cols=0)
    x = _calib(t, n, seed=t + n, outliers=6)
    qw, s, best, losses = producers.awq(to_dev(w), to_dev(x), g, bits, sym, grid)
    torch.cuda.synchronize()
    mean = orc.awq_act_mean(x.view(np.uint16))
    want_losses, want = [], None
    for i in range(grid + 1):
        si = orc.awq_scales(mean, i / grid)
        p, sc, z, w_eff = orc.awq_apply(w, si, g, bits, sym)
        loss = orc.awq_loss(x.view(np.uint16), w, w_eff)
        want_losses.append(loss)
        if want is None or loss < want[1]:
            want = (i, loss, si, p, sc, z)
    _eq(losses, np.array(want_losses, dtype=np.float32), "errors")
    assert int(best.item()) == want[0]
    _eq(s, want[2], "s")
    _eq(u32_bits(qw.qweight), want[3], "codes")
    _eq(f16_bits(qw.scales), want[4], "scales")
    _eq(f16_bits(qw.zeros), want[5], "zeros")
