"""One parity case per kernel configuration the linear-layer dispatch rules
can reach (tests/linear_cases.py, COVERAGE; a CPU test checks that the list
covers every reachable configuration).  Each case quantizes on the GPU,
compares the packed codes of the checked rows with the oracle bit for bit and
y within |y - y_ref| <= 2e-3 sum|x w'| + 1e-5 against the oracle's binary64
product."""
import numpy as np
import pytest
import torch

import w4a16_dequant_gemv_amd as w4
from gpu_util import assert_bits_equal, assert_within_tolerance, f16_bits, u32_bits, realign_metadata
from linear_cases import COVERAGE
from w4a16_dequant_gemv_amd import synthetic

pytestmark = pytest.mark.gpu


def case_id(c):
    return f"{c.kind}-int{c.bits}-m{c.m}-{c.n_out}x{c.n_in}-g{c.group_size}-a{c.align % 16}"


def run_case(orc, c, seed):
    """Quantize, run, and check the case; rows are all of them for small
    matrices, else 384 sampled rows plus the last 20."""
    dev = torch.device("cuda:0")
    print(f"case {case_id(c)} config={w4.kernel_config(c.kind, c.bits, c.m, c.n_out, c.n_in, c.group_size, c.align, c.align)}",
          flush=True)
    w_dev = synthetic.normal_weight_device(c.n_out, c.n_in, seed, 0.02, synthetic.n_outliers(c.n_in), dev)
    x = synthetic.activations_f16(c.m, c.n_in, seed=seed + 1)
    qw = w4.quantize_pack(w_dev, c.group_size, bits=c.bits)
    qw = realign_metadata(qw, c.align)
    assert qw.scales.data_ptr() % 16 == c.align % 16 and qw.zeros.data_ptr() % 16 == c.align % 16
    fn = w4.gemv if c.kind == "gemv" else w4.gemm
    y = fn(torch.from_numpy(x).to(dev), qw)
    torch.cuda.synchronize()
    if c.n_out <= 4096:
        rows = np.arange(c.n_out)
    else:
        rows = np.random.default_rng(seed).choice(c.n_out, size=384, replace=False)
        rows = np.unique(np.concatenate([rows, np.arange(c.n_out - 20, c.n_out)]))
    idx = torch.from_numpy(rows).to(dev)
    w_rows = w_dev[idx].cpu().numpy()
    del w_dev
    packed, scales, zeros, _ = orc.quantize_pack(w_rows, c.group_size, bits=c.bits)
    assert_bits_equal(u32_bits(qw.qweight[idx]), packed, f"{case_id(c)} packed")
    assert_bits_equal(f16_bits(qw.scales[idx]), scales, f"{case_id(c)} scales")
    assert_bits_equal(f16_bits(qw.zeros[idx]), zeros, f"{case_id(c)} zeros")
    y_ref, a_ref = orc.linear_from_packed(x.view(np.uint16), packed, scales, zeros, c.group_size, bits=c.bits)
    assert_within_tolerance(y[:, idx], y_ref, a_ref, case_id(c))


@pytest.mark.parametrize("case", COVERAGE, ids=case_id)
def test_every_kernel_configuration(orc, case):
    run_case(orc, case, seed=case.n_out * 31 + case.n_in + case.m + case.bits)
