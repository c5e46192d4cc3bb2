"""The C-ABI library loads, exports every symbol the header declares, and
rejects bad arguments before touching the GPU (runs without a GPU).

Every call here carries at least one invalid argument, so no kernel is ever
launched with the placeholder pointers used below.
"""
import ctypes
import os
import re

import pytest

from w4a16_dequant_gemv_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "w4a16.h")
HEADERS = [HEADER] + [os.path.join(ROOT, "include", h) for h in ("kv_codec.h", "w8a8.h", "producers.h")]

P16 = 0x10000      # 16-byte aligned placeholder address (never dereferenced)
P2 = 0x10002       # 2-byte but not 16-byte aligned


def header_functions():
    names = set()
    for h in HEADERS:
        text = open(h, encoding="utf-8").read()
        names |= set(re.findall(r"^\s*(?:int64_t|int|const char \*)\s*((?:q[48]|kv|sq|w8a8|gptq|awq)_\w+)\s*\(",
                                text, re.M))
    return sorted(names)


@pytest.fixture(scope="module")
def L():
    return _lib.lib()


def test_every_declared_symbol_is_exported(L):
    names = header_functions()
    assert set(names) == set(_lib.SIGNATURES), names
    for n in names:
        assert hasattr(L, n)


def test_version_and_strerror(L):
    assert L.q4_abi_version() == _lib.ABI_VERSION
    text = open(HEADER, encoding="utf-8").read()
    assert int(re.search(r"#define Q4_ABI_VERSION (\d+)", text).group(1)) == _lib.ABI_VERSION
    for code in range(6):
        assert L.q4_strerror(code)
    assert L.q4_strerror(0) == b"success"
    assert b"unknown" in L.q4_strerror(99)
    assert L.q4_last_hip_error() == 0


def _gemv_args(**kw):
    a = dict(x=P16, qw=P16, s=P2, z=P2, m=1, n_out=64, n_in=256, g=128, y=P2)
    a.update(kw)
    return (a["x"], a["qw"], a["s"], a["z"], a["m"], a["n_out"], a["n_in"], a["g"], a["y"], None)


@pytest.mark.parametrize("fn", ["q4_gemv", "q4_gemm"])
@pytest.mark.parametrize("bad,code", [
    (dict(x=None), _lib.Q4_ERR_NULL), (dict(qw=None), _lib.Q4_ERR_NULL),
    (dict(s=None), _lib.Q4_ERR_NULL), (dict(z=None), _lib.Q4_ERR_NULL),
    (dict(y=None), _lib.Q4_ERR_NULL),
    (dict(m=0), _lib.Q4_ERR_SHAPE), (dict(m=-1), _lib.Q4_ERR_SHAPE),
    (dict(n_out=0), _lib.Q4_ERR_SHAPE), (dict(n_in=0), _lib.Q4_ERR_SHAPE),
    (dict(n_in=-128), _lib.Q4_ERR_SHAPE),
    (dict(n_in=200), _lib.Q4_ERR_SHAPE),             # not a multiple of g
    (dict(n_in=1 << 21), _lib.Q4_ERR_SHAPE),         # beyond the n_in limit
    (dict(n_out=1 << 25), _lib.Q4_ERR_SHAPE),
    (dict(g=48), _lib.Q4_ERR_GROUP), (dict(g=0), _lib.Q4_ERR_GROUP),
    (dict(g=512), _lib.Q4_ERR_GROUP), (dict(g=16), _lib.Q4_ERR_GROUP),
    (dict(x=P16 + 8), _lib.Q4_ERR_ALIGN), (dict(qw=P16 + 4), _lib.Q4_ERR_ALIGN),
    (dict(s=P16 + 1), _lib.Q4_ERR_ALIGN), (dict(y=P16 + 1), _lib.Q4_ERR_ALIGN),
])
def test_linear_rejects(L, fn, bad, code):
    assert getattr(L, fn)(*_gemv_args(**bad)) == code


def test_gemv_rejects_more_than_16_rows(L):
    assert L.q4_gemv(*_gemv_args(m=17, x=None)) == _lib.Q4_ERR_NULL
    assert L.q4_gemv(*_gemv_args(m=17, g=48)) == _lib.Q4_ERR_GROUP
    assert L.q4_gemv(*_gemv_args(m=17, n_in=0)) == _lib.Q4_ERR_SHAPE
    # m = 17 with otherwise valid arguments must be a shape error for gemv;
    # an unaligned y keeps gemm from launching if the m rule were missing.
    assert L.q4_gemv(*_gemv_args(m=17, y=P16 + 1)) == _lib.Q4_ERR_SHAPE


@pytest.mark.parametrize("bad,code", [
    (dict(w=None), _lib.Q4_ERR_NULL), (dict(q=None), _lib.Q4_ERR_NULL),
    (dict(s=None), _lib.Q4_ERR_NULL), (dict(z=None), _lib.Q4_ERR_NULL),
    (dict(n_out=0), _lib.Q4_ERR_SHAPE), (dict(n_in=96, g=64), _lib.Q4_ERR_SHAPE),
    (dict(g=100), _lib.Q4_ERR_GROUP), (dict(w=P16 + 4), _lib.Q4_ERR_ALIGN),
    (dict(q=P16 + 8), _lib.Q4_ERR_ALIGN), (dict(z=P16 + 1), _lib.Q4_ERR_ALIGN),
])
def test_quantize_rejects(L, bad, code):
    a = dict(w=P16, n_out=8, n_in=256, g=128, sym=0, q=P16, s=P2, z=P2)
    a.update(bad)
    assert L.q4_quantize_pack(a["w"], a["n_out"], a["n_in"], a["g"], a["sym"], a["q"], a["s"],
                              a["z"], None) == code


@pytest.mark.parametrize("bad,code", [
    (dict(q=None), _lib.Q4_ERR_NULL), (dict(out=None), _lib.Q4_ERR_NULL),
    (dict(n_in=-256), _lib.Q4_ERR_SHAPE), (dict(g=8), _lib.Q4_ERR_GROUP),
    (dict(out=P16 + 4), _lib.Q4_ERR_ALIGN), (dict(s=P16 + 1), _lib.Q4_ERR_ALIGN),
])
def test_dequant_rejects(L, bad, code):
    a = dict(q=P16, s=P2, z=P2, n_out=8, n_in=256, g=128, out=P16)
    a.update(bad)
    assert L.q4_dequant(a["q"], a["s"], a["z"], a["n_out"], a["n_in"], a["g"], a["out"],
                        None) == code


def test_python_api_refuses_cpu_tensors():
    import torch
    import w4a16_dequant_gemv_amd as w4
    with pytest.raises(w4.W4A16Error):
        w4.quantize_pack(torch.zeros(4, 128), 128)
    with pytest.raises(w4.W4A16Error):
        w4.quantize_pack(torch.zeros(4, 100), 50)


def test_no_allocation_calls_in_the_boundary():
    """The library allocates nothing: no hipMalloc/hipFree in its sources."""
    csrc = os.path.join(ROOT, "w4a16_dequant_gemv_amd", "csrc")
    for f in os.listdir(csrc):
        text = open(os.path.join(csrc, f), encoding="utf-8").read()
        assert "hipMalloc" not in text and "hipFree" not in text, f
        assert "hipDeviceSynchronize" not in text and "hipStreamSynchronize" not in text, f


def _qp_args(**kw):
    a = dict(w=P16, n_out=8, n_in=256, g=128, sym=0, qw=P16, s=P2, z=P2)
    a.update(kw)
    return (a["w"], a["n_out"], a["n_in"], a["g"], a["sym"], a["qw"], a["s"], a["z"], None)


@pytest.mark.parametrize("fn", ["q4_quantize_pack", "q8_quantize_pack"])
def test_quantize_pack_rejects(L, fn):
    f = getattr(L, fn)
    assert f(*_qp_args(w=None)) == _lib.Q4_ERR_NULL
    assert f(*_qp_args(g=48)) == _lib.Q4_ERR_GROUP
    assert f(*_qp_args(n_in=100, g=100)) == _lib.Q4_ERR_GROUP          # per-channel needs n_in % 32 == 0
    assert f(*_qp_args(n_in=0)) == _lib.Q4_ERR_SHAPE
    assert f(*_qp_args(n_in=96, g=64)) == _lib.Q4_ERR_SHAPE            # 64 does not divide 96
    assert f(*_qp_args(w=P2)) == _lib.Q4_ERR_ALIGN
    # per-channel groups of any multiple-of-32 length are accepted: the
    # first error is then the null pointer, not the group size
    assert f(*_qp_args(n_in=96, g=96, qw=None)) == _lib.Q4_ERR_NULL
    assert f(*_qp_args(n_in=11008, g=11008, w=P2)) == _lib.Q4_ERR_ALIGN


@pytest.mark.parametrize("fn", ["q4_dequant", "q8_dequant"])
def test_dequant_rejects(L, fn):
    f = getattr(L, fn)
    args = dict(qw=P16, s=P2, z=P2, n_out=8, n_in=256, g=128, out=P16)
    def call(**kw):
        a = dict(args); a.update(kw)
        return f(a["qw"], a["s"], a["z"], a["n_out"], a["n_in"], a["g"], a["out"], None)
    assert call(out=None) == _lib.Q4_ERR_NULL
    assert call(g=512) == _lib.Q4_ERR_GROUP
    assert call(out=P2) == _lib.Q4_ERR_ALIGN
    assert call(n_in=160, g=160, qw=None) == _lib.Q4_ERR_NULL


@pytest.mark.parametrize("fn", ["q4_gemv", "q4_gemm"])
def test_linear_accepts_per_channel_groups(L, fn):
    f = getattr(L, fn)
    assert f(*_gemv_args(n_in=11008, g=11008, x=None)) == _lib.Q4_ERR_NULL
    assert f(*_gemv_args(n_in=11008, g=11000)) == _lib.Q4_ERR_GROUP


def _kv_tok(**kw):
    a = dict(x=P16, rows=64, d=128, bits=8, q=P16, s=P16)
    a.update(kw)
    return (a["x"], a["rows"], a["d"], a["bits"], a["q"], a["s"], None)


@pytest.mark.parametrize("bad,code", [
    (dict(x=None), _lib.Q4_ERR_NULL), (dict(q=None), _lib.Q4_ERR_NULL), (dict(s=None), _lib.Q4_ERR_NULL),
    (dict(rows=0), _lib.Q4_ERR_SHAPE), (dict(d=0), _lib.Q4_ERR_SHAPE), (dict(d=100), _lib.Q4_ERR_SHAPE),
    (dict(d=520), _lib.Q4_ERR_SHAPE), (dict(bits=6), _lib.Q4_ERR_SHAPE), (dict(bits=16), _lib.Q4_ERR_SHAPE),
    (dict(x=P16 + 8), _lib.Q4_ERR_ALIGN), (dict(q=P16 + 8), _lib.Q4_ERR_ALIGN), (dict(s=P16 + 2), _lib.Q4_ERR_ALIGN),
])
def test_kv_quant_tokens_rejects(L, bad, code):
    assert L.kv_quant_tokens(*_kv_tok(**bad)) == code


def _kv_ch(**kw):
    a = dict(x=P16, blocks=4, t=128, d=128, bits=8, q=P16, s=P16)
    a.update(kw)
    return (a["x"], a["blocks"], a["t"], a["d"], a["bits"], a["q"], a["s"], None)


@pytest.mark.parametrize("bad,code", [
    (dict(x=None), _lib.Q4_ERR_NULL), (dict(blocks=0), _lib.Q4_ERR_SHAPE), (dict(t=0), _lib.Q4_ERR_SHAPE),
    (dict(t=513), _lib.Q4_ERR_SHAPE),               # beyond 32 rows per thread at d = 128
    (dict(d=256, t=257), _lib.Q4_ERR_SHAPE), (dict(d=12), _lib.Q4_ERR_SHAPE), (dict(bits=3), _lib.Q4_ERR_SHAPE),
    (dict(x=P16 + 2), _lib.Q4_ERR_ALIGN), (dict(s=P16 + 1), _lib.Q4_ERR_ALIGN),
])
def test_kv_quant_channels_rejects(L, bad, code):
    assert L.kv_quant_channels(*_kv_ch(**bad)) == code


def test_kv_limits_accept_the_extremes(L):
    # the largest t at each d passes the shape rules (the null output is the first error)
    for d, t in ((8, 8192), (64, 1024), (128, 512), (256, 256), (512, 128)):
        assert L.kv_quant_channels(*_kv_ch(d=d, t=t, q=None)) == _lib.Q4_ERR_NULL
        assert L.kv_quant_channels(*_kv_ch(d=d, t=t + 1, q=None)) == _lib.Q4_ERR_NULL
        assert L.kv_quant_channels(*_kv_ch(d=d, t=t + 1)) == _lib.Q4_ERR_SHAPE


def test_kv_dequant_rejects(L):
    assert L.kv_dequant_tokens(None, P16, 4, 128, P16, None) == _lib.Q4_ERR_NULL
    assert L.kv_dequant_tokens(P16, P16, 4, 132, P16, None) == _lib.Q4_ERR_SHAPE
    assert L.kv_dequant_tokens(P16, P16, 4, 128, P16 + 2, None) == _lib.Q4_ERR_ALIGN
    assert L.kv_dequant_channels(P16, P16, 4, 128, 128, None, None) == _lib.Q4_ERR_NULL
    assert L.kv_dequant_channels(P16, P16 + 4, 4, 128, 128, P16, None) == _lib.Q4_ERR_ALIGN
    assert L.kv_dequant_channels(P16, P16, 4, 0, 128, P16, None) == _lib.Q4_ERR_SHAPE


def test_kv_flush_rejects(L):
    def call(**kw):
        a = dict(k=P16, v=P16, blocks=4, t=128, d=128, bits=8, dst=P16, pool=16, kp=P16, ks=P16, vp=P16, vs=P16)
        a.update(kw)
        return L.kv_flush_blocks(a["k"], a["v"], a["blocks"], a["t"], a["d"], a["bits"], a["dst"], a["pool"],
                                 a["kp"], a["ks"], a["vp"], a["vs"], None)
    assert call(dst=None) == _lib.Q4_ERR_NULL
    assert call(vs=None) == _lib.Q4_ERR_NULL
    assert call(pool=0) == _lib.Q4_ERR_SHAPE
    assert call(bits=5) == _lib.Q4_ERR_SHAPE
    assert call(dst=P16 + 2) == _lib.Q4_ERR_ALIGN
    assert call(vp=P16 + 4) == _lib.Q4_ERR_ALIGN


def test_w8a8_rejects(L):
    # calibration maxima
    assert L.sq_absmax_update_f16(None, 4, 64, P16, None) == _lib.Q4_ERR_NULL
    assert L.sq_absmax_update_f16(P16, 4, 60, P16, None) == _lib.Q4_ERR_SHAPE
    assert L.sq_absmax_update_f32(P16, 0, 64, P16, None) == _lib.Q4_ERR_SHAPE
    assert L.sq_absmax_update_f32(P16 + 4, 4, 64, P16, None) == _lib.Q4_ERR_ALIGN
    # factors
    assert L.sq_smooth_factors(P16, P16, 64, 1.5, P16, None) == _lib.Q4_ERR_SHAPE
    assert L.sq_smooth_factors(P16, P16, 64, float("nan"), P16, None) == _lib.Q4_ERR_SHAPE
    assert L.sq_smooth_factors(P16, None, 64, 0.5, P16, None) == _lib.Q4_ERR_NULL
    # quantizers: k a multiple of 32 in [32, 32768]
    assert L.w8a8_quantize_weight(P16, None, 8, 100, P16, P16, None) == _lib.Q4_ERR_SHAPE
    assert L.w8a8_quantize_weight(P16, None, 8, 32800, P16, P16, None) == _lib.Q4_ERR_SHAPE
    assert L.w8a8_quantize_weight(P16, P16 + 4, 8, 96, P16, P16, None) == _lib.Q4_ERR_ALIGN
    assert L.w8a8_quantize_act(P16, None, 0, 96, P16, P16, None) == _lib.Q4_ERR_SHAPE
    assert L.w8a8_quantize_act(P16 + 2, None, 4, 96, P16, P16, None) == _lib.Q4_ERR_ALIGN
    assert L.w8a8_quantize_act(P16, None, 4, 96, None, P16, None) == _lib.Q4_ERR_NULL
    # product
    assert L.w8a8_gemm(P16, P16, P16, P16, 4, 8, 48, P16, None) == _lib.Q4_ERR_SHAPE
    assert L.w8a8_gemm(P16, P16, P16, P16, 4, 0, 64, P16, None) == _lib.Q4_ERR_SHAPE
    assert L.w8a8_gemm(P16 + 8, P16, P16, P16, 4, 8, 64, P16, None) == _lib.Q4_ERR_ALIGN
    assert L.w8a8_gemm(P16, P16, P16, P16, 4, 8, 64, P16 + 1, None) == _lib.Q4_ERR_ALIGN
    assert L.w8a8_gemm(P16, None, P16, P16, 4, 8, 64, P16, None) == _lib.Q4_ERR_NULL


def test_producers_reject(L):
    assert L.gptq_factor_workspace_size(256) == 2 * 256 * 256 * 8
    assert L.gptq_hinv_factor(P16, 64, 256, 0.01, None, 1 << 20, P16, None) == _lib.Q4_ERR_NULL
    assert L.gptq_hinv_factor(P16, 64, 100, 0.01, P16, 1 << 20, P16, None) == _lib.Q4_ERR_SHAPE
    assert L.gptq_hinv_factor(P16, 64, 256, 0.01, P16, 1000, P16, None) == _lib.Q4_ERR_SHAPE   # workspace too small
    assert L.gptq_hinv_factor(P16, 64, 256, -1.0, P16, 1 << 20, P16, None) == _lib.Q4_ERR_SHAPE
    assert L.gptq_hinv_factor(P16, 64, 256, 0.01, P16 + 16, 1 << 20, P16, None) == _lib.Q4_ERR_ALIGN
    ws = L.gptq_quantize_workspace_size(8, 256)
    assert L.gptq_quantize(P16, P16, 8, 256, 48, 4, 0, P16, ws, P16, P2, P2, None) == _lib.Q4_ERR_GROUP
    assert L.gptq_quantize(P16, P16, 8, 256, 128, 3, 0, P16, ws, P16, P2, P2, None) == _lib.Q4_ERR_SHAPE
    assert L.gptq_quantize(P16, P16, 8, 256, 128, 4, 0, P16, ws - 1, P16, P2, P2, None) == _lib.Q4_ERR_SHAPE
    assert L.gptq_quantize(P16, P16, 8, 256, 128, 4, 0, P16, ws, P16 + 4, P2, P2, None) == _lib.Q4_ERR_ALIGN
    # the no-allocation column loop: the same checks, and its fixed capacity
    assert L.gptq_quantize_noalloc(P16, P16, 8, 256, 48, 4, 0, P16, P2, P2, None) == _lib.Q4_ERR_GROUP
    assert L.gptq_quantize_noalloc(P16, None, 8, 256, 128, 4, 0, P16, P2, P2, None) == _lib.Q4_ERR_NULL
    assert L.gptq_quantize_noalloc(P16 + 4, P16, 8, 256, 128, 4, 0, P16, P2, P2, None) == _lib.Q4_ERR_ALIGN
    assert L.gptq_quantize_workspace_size(4096, 4096) <= L.gptq_quantize_noalloc_max_bytes() == 72 << 20
    assert L.gptq_quantize_noalloc(P16, P16, 4096, 4608, 128, 4, 0, P16, P2, P2, None) == _lib.Q4_ERR_CAPACITY
    wa = L.awq_workspace_size(8, 256, 64, 20, 128)
    assert wa > 0
    assert L.awq_quantize(P16, P16, 64, 8, 256, 128, 4, 0, 0, P16, wa, P16, P2, P2, P16, None, None, None) == _lib.Q4_ERR_SHAPE
    assert L.awq_quantize(P16, P16, 64, 8, 256, 128, 4, 0, 20, P16, wa - 1, P16, P2, P2, P16, None, None, None) == _lib.Q4_ERR_SHAPE
    assert L.awq_quantize(P16, P16, 64, 8, 256, 128, 4, 0, 20, P16, wa, P16, P2, P2, None, None, None, None) == _lib.Q4_ERR_NULL
