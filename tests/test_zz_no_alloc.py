"""gptq_quantize_noalloc -- the GPTQ column loop with no workspace argument and
no allocation (its scratch is a fixed array the library holds per GPU) --
against gptq_quantize with a caller workspace, bit for bit, called through
the C ABI: two calls in a row (the second smaller, on the scratch the first
left behind), the largest layer shape the scratch is sized for, and the
capacity error for a larger one."""
import ctypes

import numpy as np
import pytest
import torch

from w4a16_dequant_gemv_amd import producers
from w4a16_dequant_gemv_amd._lib import Q4_ERR_CAPACITY, lib

pytestmark = pytest.mark.gpu


def _weights(n_out, n, seed):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    return (torch.randn((n_out, n), generator=g, device="cuda") * 0.02).contiguous()


def _factor(n, tokens, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((tokens, n)).astype(np.float32)
    x[:, rng.choice(n, 3, replace=False)] *= 8.0
    return producers.gptq_factor(torch.from_numpy(x.astype(np.float16)).cuda())


def _noalloc(w, u, g, bits, sym):
    n_out, n = w.shape
    out = producers._outputs(n_out, n, g, bits, sym, w.device)
    stream = torch.cuda.current_stream().cuda_stream
    rc = lib().gptq_quantize_noalloc(w.data_ptr(), u.data_ptr(), n_out, n, g, bits, int(sym),
                                     out.qweight.data_ptr(), out.scales.data_ptr(), out.zeros.data_ptr(), stream)
    assert rc == 0, rc
    torch.cuda.synchronize()
    return out


def _same(a, b, what):
    for name in ("qweight", "scales", "zeros"):
        x, y = getattr(a, name), getattr(b, name)
        assert torch.equal(x.view(torch.int16) if x.dtype == torch.float16 else x,
                           y.view(torch.int16) if y.dtype == torch.float16 else y), f"{what}: {name} differs"


def test_noalloc_matches_workspace_entry_point_on_consecutive_calls():
    cases = [(512, 1024, 128, 4, False, 1), (96, 256, 32, 8, True, 2)]      # the second is smaller
    for n_out, n, g, bits, sym, seed in cases:
        print(f"gptq_quantize_noalloc n_out={n_out} n={n} g={g} bits={bits} sym={sym}", flush=True)
        w = _weights(n_out, n, seed)
        u = _factor(n, 256, seed + 10)
        ref = producers.gptq_quantize(w, u, g, bits, sym)
        torch.cuda.synchronize()
        got = _noalloc(w, u, g, bits, sym)
        _same(got, ref, f"{n_out}x{n} g={g} bits={bits} sym={sym}")


def test_noalloc_largest_supported_layer():
    n_out, n = 4096, 4096
    assert lib().gptq_quantize_workspace_size(n_out, n) <= lib().gptq_quantize_noalloc_max_bytes()
    print(f"gptq_quantize_noalloc n_out={n_out} n={n}", flush=True)
    w = _weights(n_out, n, 3)
    u = _factor(n, 512, 13)
    ref = producers.gptq_quantize(w, u, 128)
    torch.cuda.synchronize()
    _same(_noalloc(w, u, 128, 4, False), ref, "4096x4096")


def test_noalloc_rejects_a_problem_beyond_its_scratch():
    n_out, n = 4096, 4608
    assert lib().gptq_quantize_workspace_size(n_out, n) > lib().gptq_quantize_noalloc_max_bytes()
    p = 1 << 20            # placeholder addresses: the call is rejected before any HIP call
    assert lib().gptq_quantize_noalloc(p, p, n_out, n, 128, 4, 0, p, p, p, None) == Q4_ERR_CAPACITY
