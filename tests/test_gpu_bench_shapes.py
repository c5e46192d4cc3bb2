"""Every linear-layer call the benchmark times, on the benchmark's own inputs
(bench.timed_linear_calls and its workload builders), against the oracle:
packed codes, scales and zero-points of the checked rows bit for bit, y
within |y - y_ref| <= 2e-3 sum|x w'| + 1e-5 against the binary64 product.

Rows checked: all of them for the 7B decode linears and the 4096x4096
linear; 512 sampled rows plus the last 20 for the 70B linears (layers 0, 40
and 79) and the 8192x28672 stress matrix; for the m = 2048 prefill shapes,
48 sampled rows of x (the first and last among them) against every output
channel."""
import numpy as np
import pytest
import torch

import bench
import w4a16_dequant_gemv_amd as w4
from gpu_util import assert_bits_equal, assert_within_tolerance, f16_bits, u32_bits
from w4a16_dequant_gemv_amd import synthetic as syn
from w4a16_dequant_gemv_amd.api import QuantizedWeight

pytestmark = pytest.mark.gpu


def call_id(c):
    return f"{c.leg}{c.index}-int{c.bits}-m{c.m}-{c.n_out}x{c.n_in}-g{c.group_size}{'-sym' if c.symmetric else ''}"


def _cases():
    out = []
    for c in bench.timed_linear_calls():
        for layer in ((0, 40, 79) if c.leg == "decode70b" else (0,)):
            for copy in ((0, bench.SINGLE_COPIES - 1) if c.leg == "single" else (0,)):
                out.append(pytest.param(c, layer, copy, id=f"{call_id(c)}-L{layer}-c{copy}"))
    return out


def _inputs(c, layer, copy, dev):
    """(fp32 weights, fp16 x) of the call, built as the benchmark builds them."""
    if c.leg in ("decode7b", "w8a16_decode"):
        return bench.decode7b_weight(layer, c.index, dev), bench.decode7b_x(c.index, dev, int8=c.bits == 8)
    if c.leg == "decode7b_split":
        j, _ = bench.split_of(c.index)
        return bench.decode7b_weight(layer, j, dev), bench.decode7b_x(j, dev)
    if c.leg == "decode70b":
        return bench.decode70b_weight(layer, c.index, dev), bench.decode70b_x(c.index, dev)
    if c.leg == "stress":
        return bench.stress_weight(c.group_size, dev), bench.stress_x(dev)
    if c.leg == "single":
        return bench.single_copy(bench.single_weight(dev), copy), bench.single_x(dev)
    if c.leg in ("prefill", "w8a16_prefill"):
        return bench.prefill_weight(c.index, dev), bench.prefill_x(c.index, dev)
    raise ValueError(c.leg)


@pytest.mark.parametrize("c,layer,copy", _cases())
def test_bench_call(orc, c, layer, copy):
    dev = torch.device("cuda:0")
    print(f"bench call {call_id(c)} layer={layer} copy={copy} "
          f"config={w4.kernel_config(c.kind, c.bits, c.m, c.n_out, c.n_in, c.group_size)}", flush=True)
    w, x = _inputs(c, layer, copy, dev)
    qw = w4.quantize_pack(w, c.group_size, c.symmetric, bits=c.bits)
    if c.leg == "decode7b_split":
        # the benchmark's per-linear launches run on row slices of the fused matrix
        _, off = bench.split_of(c.index)
        sl = slice(off, off + c.n_out)
        qw = QuantizedWeight(qw.qweight[sl], qw.scales[sl], qw.zeros[sl], c.n_out, c.n_in, c.group_size)
        w = w[sl]
    assert (qw.n_out, qw.n_in) == (c.n_out, c.n_in) and tuple(x.shape) == (c.m, c.n_in)
    fn = w4.gemv if c.kind == "gemv" else w4.gemm
    y = fn(x, qw)
    torch.cuda.synchronize()
    rng = np.random.default_rng(c.n_out + layer + copy)
    if c.kind == "gemm":
        xrows = np.sort(rng.choice(c.m, 48, replace=False))
        xrows[0], xrows[-1] = 0, c.m - 1
        rows = np.arange(c.n_out)
    else:
        xrows = np.arange(c.m)
        if c.leg in ("decode70b", "stress"):
            rows = np.unique(np.concatenate([rng.choice(c.n_out, 512, replace=False),
                                             np.arange(c.n_out - 20, c.n_out)]))
        else:
            rows = np.arange(c.n_out)
    idx = torch.from_numpy(rows).to(dev)
    w_rows = w[idx].cpu().numpy()
    del w
    packed, scales, zeros, _ = orc.quantize_pack(w_rows, c.group_size, c.symmetric, bits=c.bits)
    what = f"{call_id(c)} layer {layer} copy {copy}"
    assert_bits_equal(u32_bits(qw.qweight[idx]), packed, f"{what} packed")
    assert_bits_equal(f16_bits(qw.scales[idx]), scales, f"{what} scales")
    assert_bits_equal(f16_bits(qw.zeros[idx]), zeros, f"{what} zeros")
    xh = x[torch.from_numpy(xrows).to(dev)].cpu().numpy()
    y_ref, a_ref = orc.linear_from_packed(xh.view(np.uint16), packed, scales, zeros, c.group_size, bits=c.bits)
    y_sel = y[torch.from_numpy(xrows).to(dev)][:, idx]
    assert_within_tolerance(y_sel, y_ref, a_ref, what)
