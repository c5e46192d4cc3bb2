"""Seeded synthetic inputs shaped like the models the pages discuss.

This module only draws random numbers; it holds none of the quantization or
matrix arithmetic.  Both the GPU path and the CPU oracle take its outputs as
plain arrays, so it is the only code the two sides share.

Distributions follow the workloads:
  * weights W[out, in] ~ N(0, std) in float32, with a small set of input
    columns scaled by 50 to stand in for outlier channels (the pages put
    such channels at about 0.1 % and 50-100x the typical range);
  * heavy-tailed weights 0.02 * Student-t(3) with a share of constant
    groups (max == min) and of all-zero groups;
  * activations x ~ N(0, 1), rounded once to fp16.
"""
from dataclasses import dataclass

import numpy as np

OUTLIER_SCALE = 50.0


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def outlier_columns(n_in, count, seed):
    """The input-dimension indices scaled as outlier channels."""
    if count <= 0:
        return np.zeros(0, dtype=np.int64)
    return np.sort(_rng(seed + 7_000_003).choice(n_in, size=count, replace=False))


def normal_weight(n_out, n_in, seed, std=0.02, n_outlier_cols=0):
    """float32 [n_out][n_in] ~ N(0, std), `n_outlier_cols` columns x50."""
    w = _rng(seed).standard_normal((n_out, n_in), dtype=np.float32)
    w *= np.float32(std)
    cols = outlier_columns(n_in, n_outlier_cols, seed)
    if cols.size:
        w[:, cols] *= np.float32(OUTLIER_SCALE)
    return w


def student_t_weight(n_out, n_in, seed, group_size, nu=3.0, scale=0.02,
                     const_frac=0.01, zero_frac=0.001):
    """float32 [n_out][n_in] = scale * t(nu); a `const_frac` share of groups is
    set to the group's first value, a `zero_frac` share to exactly 0."""
    rng = _rng(seed)
    w = (rng.standard_t(nu, size=(n_out, n_in)) * scale).astype(np.float32)
    groups = w.reshape(n_out, n_in // group_size, group_size)
    total = groups.shape[0] * groups.shape[1]
    flat = groups.reshape(total, group_size)
    n_const = int(round(const_frac * total))
    n_zero = int(round(zero_frac * total))
    pick = rng.choice(total, size=n_const + n_zero, replace=False)
    flat[pick[:n_const]] = flat[pick[:n_const], :1]
    flat[pick[n_const:]] = 0.0
    return w


def activations_f16(m, n_in, seed):
    """fp16 [m][n_in] ~ N(0, 1) (drawn in float32, rounded to fp16 once)."""
    return _rng(seed).standard_normal((m, n_in), dtype=np.float32).astype(np.float16)


# ---------------------------------------------------------------------------
# GPU-side generators for workloads too large to draw on the host.  They use
# torch's seeded device generator; parity tests copy the rows they check back
# to the host.
# ---------------------------------------------------------------------------

def normal_weight_device(n_out, n_in, seed, std, n_outlier_cols, device):
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    w = torch.randn((n_out, n_in), generator=gen, device=device, dtype=torch.float32)
    w.mul_(std)
    cols = outlier_columns(n_in, n_outlier_cols, seed)
    if cols.size:
        idx = torch.from_numpy(cols).to(device)
        w[:, idx] *= OUTLIER_SCALE
    return w


def student_t_weight_device(n_out, n_in, seed, group_size, device, nu=3, scale=0.02,
                            const_frac=0.01, zero_frac=0.001):
    """float32 [n_out][n_in] = scale * t(nu) on the GPU (t drawn as
    N(0,1) / sqrt(chi2(nu) / nu), nu an integer); a `const_frac` share of the
    groups of `group_size` is set to the group's first value and a
    `zero_frac` share to exactly 0 (group indices drawn on the host)."""
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    w = torch.randn((n_out, n_in), generator=gen, device=device, dtype=torch.float32)
    chi2 = torch.zeros_like(w)
    for _ in range(nu):
        e = torch.randn((n_out, n_in), generator=gen, device=device, dtype=torch.float32)
        chi2.addcmul_(e, e)
        del e
    w.mul_(torch.rsqrt(chi2.div_(float(nu)))).mul_(scale)
    del chi2
    groups = w.view(n_out * (n_in // group_size), group_size)
    total = groups.shape[0]
    n_const = int(round(const_frac * total))
    n_zero = int(round(zero_frac * total))
    pick = torch.from_numpy(_rng(seed).choice(total, size=n_const + n_zero, replace=False)).to(device)
    const_rows = pick[:n_const]
    groups[const_rows] = groups[const_rows, :1].expand(-1, group_size)
    groups[pick[n_const:]] = 0.0
    return w


def activations_f16_device(m, n_in, seed, device):
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    return torch.randn((m, n_in), generator=gen, device=device,
                       dtype=torch.float32).half()


def kv_values_device(shape, seed, device, n_outlier_channels=4, outlier_scale=20.0):
    """fp16 cache values [..., d] ~ N(0, 1) on the GPU with n_outlier_channels
    fixed channels (the same in every token) scaled by outlier_scale: the
    channel-wise outliers that keys carry."""
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    x = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    d = shape[-1]
    chans = _rng(seed).choice(d, size=min(n_outlier_channels, d), replace=False)
    x[..., torch.from_numpy(np.sort(chans)).to(device)] *= outlier_scale
    return x.half()


# ---------------------------------------------------------------------------
# Workload shapes.
# ---------------------------------------------------------------------------

@dataclass(frozen=True)
class Linear:
    name: str
    n_out: int
    n_in: int


# Llama-2-7B-shaped decoder layer: attention projections and the gated MLP.
LLAMA7B_LINEARS = (
    Linear("q", 4096, 4096), Linear("k", 4096, 4096), Linear("v", 4096, 4096),
    Linear("o", 4096, 4096), Linear("gate", 11008, 4096), Linear("up", 11008, 4096),
    Linear("down", 4096, 11008),
)
LLAMA7B_LAYERS = 32

# 70B-shaped decoder layer (grouped-query attention: 8 KV heads of 128).
LLAMA70B_LINEARS = (
    Linear("q", 8192, 8192), Linear("k", 1024, 8192), Linear("v", 1024, 8192),
    Linear("o", 8192, 8192), Linear("gate", 28672, 8192), Linear("up", 28672, 8192),
    Linear("down", 8192, 28672),
)
LLAMA70B_LAYERS = 80

# Prefill GEMM shapes (7B projections), M = 2048 tokens.
PREFILL_M = 2048
PREFILL_LINEARS = (Linear("qkvo", 4096, 4096), Linear("gate_up", 11008, 4096),
                   Linear("down", 4096, 11008))


# Serving engines store q, k and v as one matrix and gate and up as another:
# a decode step then runs four dependent linear layers per decoder layer
# (quantization is per row, so this equals quantizing each linear alone).
FUSED_LAYOUT = (("qkv", (0, 1, 2)), ("o", (3,)), ("gate_up", (4, 5)), ("down", (6,)))


def fused_linears(linears):
    """The four fused linears of a layer, in decode order."""
    return tuple(Linear(name, sum(linears[i].n_out for i in idx), linears[idx[0]].n_in)
                 for name, idx in FUSED_LAYOUT)


def llama7b_seed(layer, index):
    return 2000 + 16 * layer + index


def llama70b_seed(layer, index):
    return 3000 + 8 * layer + index


def n_outliers(n_in):
    """About 0.1 % of the input columns."""
    return int(round(0.001 * n_in))

# KV cache of one Llama-3-70B-shaped layer (80 layers, 8 KV heads of 128 under
# grouped-query attention) at batch 32 and 32768 tokens; blocks of 128 tokens
# leave the FP16 window together.
KV70B = dict(batch=32, kv_heads=8, seq=32768, head_dim=128, block=128, layers=80)

