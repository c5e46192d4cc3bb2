"""KV-cache codec on the GPU against the CPU oracle, bit for bit: per-token
(V) and per-channel (K) quantization, both dequantizations, and the flush of
window blocks into a block pool."""
import numpy as np
import pytest
import torch

from gpu_util import to_dev
from w4a16_dequant_gemv_amd import kv, synthetic

pytestmark = pytest.mark.gpu


def _kv_values(shape, seed, outlier_channels=2):
    """fp16 [..., d] ~ N(0, 1) with a few x40 channels, an all-zero token,
    a constant token, tiny (subnormal) and extreme values."""
    rng = np.random.default_rng(seed)
    a = rng.standard_normal(shape).astype(np.float32)
    d = shape[-1]
    flat = a.reshape(-1, d)
    for c in rng.choice(d, size=min(outlier_channels, d), replace=False):
        flat[:, c] *= 40.0
    if flat.shape[0] > 3:
        flat[1] = 0.0
        flat[2] = -0.75
        flat[3] = rng.standard_normal(d).astype(np.float32) * 3e-7      # fp16 subnormals
    if flat.shape[0] > 4:
        flat[4, 0] = 65504.0
        flat[4, -1] = -65504.0
    return flat.reshape(shape).astype(np.float16)


def _eq(got, want, what):
    got = got.cpu().numpy()
    assert got.shape == want.shape, (what, got.shape, want.shape)
    if got.dtype == np.float32:
        got, want = got.view(np.uint32), want.view(np.uint32)
    bad = np.argwhere(got != want)
    assert bad.size == 0, f"{what}: {len(bad)} mismatches, first at {bad[:3].tolist()}"


@pytest.mark.parametrize("bits", [8, 4])
@pytest.mark.parametrize("rows,d", [(1, 8), (3, 64), (1000, 128), (257, 80), (64, 256), (33, 512), (5, 96)])
def test_quant_tokens_bit_exact(orc, bits, rows, d):
    x = _kv_values((rows, d), seed=rows * 7 + d)
    q, s = kv.quant_tokens(to_dev(x), bits)
    torch.cuda.synchronize()
    q_ref, s_ref = orc.kv_quant_tokens(x.view(np.uint16), bits)
    _eq(q, q_ref, f"codes rows={rows} d={d} b{bits}")
    _eq(s, s_ref, f"scales rows={rows} d={d} b{bits}")
    back = kv.dequant_tokens(q, s)
    torch.cuda.synchronize()
    _eq(back.view(torch.int16), orc.kv_dequant_tokens(q_ref, s_ref).view(np.int16), "dequant")


@pytest.mark.parametrize("bits", [8, 4])
@pytest.mark.parametrize("blocks,t,d", [(1, 1, 8), (3, 128, 128), (2, 37, 80), (5, 256, 256), (2, 128, 512),
                                        (1, 8192, 8), (4, 1024, 64), (7, 512, 128), (3, 25, 128)])
def test_quant_channels_bit_exact(orc, bits, blocks, t, d):
    x = _kv_values((blocks, t, d), seed=blocks * 11 + t + d)
    q, s = kv.quant_channels(to_dev(x), bits)
    torch.cuda.synchronize()
    q_ref, s_ref = orc.kv_quant_channels(x.view(np.uint16), bits)
    _eq(q, q_ref, f"codes {blocks}x{t}x{d} b{bits}")
    _eq(s, s_ref, f"scales {blocks}x{t}x{d} b{bits}")
    back = kv.dequant_channels(q, s)
    torch.cuda.synchronize()
    _eq(back.view(torch.int16), orc.kv_dequant_channels(q_ref, s_ref).view(np.int16), "dequant")


def test_quant_tokens_4d_cache_layout(orc):
    """A [B, H, S, D] cache is B*H*S token rows."""
    x = _kv_values((2, 4, 48, 128), seed=5)
    q, s = kv.quant_tokens(to_dev(x), 8)
    torch.cuda.synchronize()
    assert tuple(s.shape) == (2, 4, 48)
    q_ref, s_ref = orc.kv_quant_tokens(x.view(np.uint16), 8)
    _eq(q, q_ref, "codes")
    _eq(s, s_ref, "scales")


@pytest.mark.parametrize("bits", [8, 4])
def test_flush_into_pool(orc, bits):
    P, t, d, pool_blocks = 9, 128, 128, 16
    kb = _kv_values((P, t, d), seed=31)
    vb = _kv_values((P, t, d), seed=32)
    dst = np.array([3, 15, -1, 0, 7, 16, 9, 2, 11], dtype=np.int32)     # -1 and 16 are skipped
    pool = kv.KVBlockPool(pool_blocks, t, d, torch.device("cuda"), bits)
    for tns in (pool.k, pool.v):
        tns.fill_(0x5A)
    pool.k_scale.fill_(-7.0)
    pool.v_scale.fill_(-7.0)
    pool.flush(to_dev(kb), to_dev(vb), to_dev(dst))
    torch.cuda.synchronize()
    want = orc.kv_flush(kb.view(np.uint16), vb.view(np.uint16), dst, pool_blocks, bits)
    named = sorted(int(s) for s in dst if 0 <= s < pool_blocks)
    for key, got in (("k", pool.k), ("k_scale", pool.k_scale), ("v", pool.v), ("v_scale", pool.v_scale)):
        _eq(got[named], want[key][named], f"pool {key}")
    untouched = [s for s in range(pool_blocks) if s not in named]
    assert (pool.k[untouched] == 0x5A).all() and (pool.v[untouched] == 0x5A).all()
    assert (pool.k_scale[untouched] == -7.0).all() and (pool.v_scale[untouched] == -7.0).all()


def test_flush_matches_separate_calls():
    """The fused flush writes what the two standalone quantizers write."""
    P, t, d = 6, 128, 128
    kb = to_dev(_kv_values((P, t, d), seed=41))
    vb = to_dev(_kv_values((P, t, d), seed=42))
    pool = kv.KVBlockPool(P, t, d, torch.device("cuda"))
    pool.flush(kb, vb, torch.arange(P, dtype=torch.int32, device="cuda"))
    qk, sk = kv.quant_channels(kb)
    qv, sv = kv.quant_tokens(vb)
    torch.cuda.synchronize()
    assert torch.equal(pool.k, qk) and torch.equal(pool.v, qv)
    assert torch.equal(pool.k_scale.view(torch.int32), sk.view(torch.int32))
    assert torch.equal(pool.v_scale.view(torch.int32), sv.view(torch.int32))


def test_llama70b_layer_cache_sampled(orc):
    """One layer of a Llama-3-70B-shaped cache (batch 32, 8 KV heads, 32768
    tokens, head dim 128; 2.1 GB of fp16 per side) in the launch shapes the
    benchmark times; sampled K blocks and V token rows against the oracle."""
    B, H, S, D, T = 32, 8, 32768, 128, 128
    dev = torch.device("cuda")
    x = synthetic.kv_values_device((B * H * S // T, T, D), seed=6100, device=dev)
    qk, sk = kv.quant_channels(x)
    qv, sv = kv.quant_tokens(x)
    torch.cuda.synchronize()
    rng = np.random.default_rng(6101)
    blocks = np.sort(rng.choice(x.shape[0], size=24, replace=False))
    blocks[0], blocks[-1] = 0, x.shape[0] - 1
    xb = x[torch.from_numpy(blocks).to(dev)].cpu().numpy().view(np.uint16)
    q_ref, s_ref = orc.kv_quant_channels(xb, 8)
    _eq(qk[torch.from_numpy(blocks).to(dev)], q_ref, "K codes")
    _eq(sk[torch.from_numpy(blocks).to(dev)], s_ref, "K scales")
    qt_ref, st_ref = orc.kv_quant_tokens(xb, 8)
    _eq(qv[torch.from_numpy(blocks).to(dev)], qt_ref, "V codes")
    _eq(sv[torch.from_numpy(blocks).to(dev)], st_ref, "V scales")
    del x, qk, sk, qv, sv
    torch.cuda.empty_cache()
