"""The GPU parity cases cover every kernel configuration the linear-layer
dispatch rules can reach, every configuration the benchmark times and every
kernel named in the committed profiles.  Runs on the CPU: the library's
kernel selection report (q4_linear_config) makes no HIP call."""
import glob
import os
import re

import pytest

from linear_cases import COVERAGE, Case, bench_cases
from w4a16_dequant_gemv_amd import api
from w4a16_dequant_gemv_amd._lib import Q4_ERR_GROUP, Q4_ERR_NULL, Q4_ERR_SHAPE, lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# Sizes around every threshold of the rules: tile counts (16 channels per
# tile) of 1, 2, 256, 257, 512, 640, 768, 769 and beyond; 128-wide k blocks
# below 16, 16..63, 64..127 and 128 or more, with and without a partial last
# block; rows of 1 to 8 chunks of 2048 codes and more; x that fits the
# LDS-resident kernels or not at every m; metadata 16- and 2-byte aligned.
N_IN = [32, 96, 128, 1024, 2016, 2048, 2080, 4096, 4224, 8192, 8320, 11008, 13312, 16384, 16416, 28672,
        32768, 65536, 131072, 262144, 1048576]
N_OUT = [16, 17, 100, 4096, 4112, 8192, 10240, 12288, 12304, 22016, 28672, 57344, 131072]
GROUPS = (32, 64, 128, 256, None)


def config(c):
    return api.kernel_config(c.kind, c.bits, c.m, c.n_out, c.n_in, c.group_size, c.align, c.align)


def cost(c):
    return c.m * c.n_in * 2 + c.n_out * c.n_in * c.bits // 8


@pytest.fixture(scope="module")
def reachable():
    out = {}
    for kind in ("gemv", "gemm"):
        for bits in (4, 8):
            for g in GROUPS:
                for n_in in N_IN:
                    gs = n_in if g is None else g
                    if n_in % gs or (kind == "gemm" and n_in > 32768):
                        continue
                    for n_out in (N_OUT if kind == "gemv" else (16, 100, 4096)):
                        if n_out * n_in > 2 ** 34:
                            continue
                        for m in (range(1, 17) if kind == "gemv" else (17, 300, 2048)):
                            aligns = ((256, 258) if m == 1 else (256,)) if kind == "gemv" else (256, 260, 258)
                            for align in aligns:
                                c = Case(kind, bits, m, n_out, n_in, gs, align)
                                try:
                                    name = config(c)
                                except api.W4A16Error:
                                    continue
                                out.setdefault(name, []).append(c)
    return out


@pytest.fixture(scope="module")
def covered():
    return {config(c) for c in COVERAGE} | {config(c) for c in bench_cases()}


def test_every_reachable_configuration_has_a_parity_case(reachable, covered):
    missing = {name: min(cases, key=cost) for name, cases in reachable.items() if name not in covered}
    assert not missing, "configurations without a GPU parity case (add one to tests/linear_cases.py): " + \
        "; ".join(f"{k}: e.g. {v}" for k, v in sorted(missing.items()))


def test_coverage_cases_are_all_reachable(reachable):
    """No stale case: each one selects a configuration the grid reaches."""
    names = set(reachable)
    stale = [c for c in COVERAGE if config(c) not in names]
    assert not stale, f"cases selecting no reachable configuration: {stale}"


def test_bench_configurations_have_parity_cases(covered):
    """Every call bench.py times runs in tests/test_gpu_bench_shapes.py on the
    benchmark's own inputs; their configurations are therefore covered."""
    cases = bench_cases()
    assert cases, "bench.timed_linear_calls() is empty"
    for c in cases:
        assert config(c) in covered


def test_profiled_kernels_are_covered(covered):
    """Every q4_gemv / q4_gemm instantiation named in a committed profile
    summary is one the parity tests run (a stale profile fails here)."""
    pat = re.compile(r"\b(gemv_resident_kernel|gemv_window_kernel|gemv_rowstream_kernel|gemv_persistent_kernel|"
                     r"gemm_kernel)<[^<>]*>")
    seen = set()
    for path in glob.glob(os.path.join(ROOT, "profiles", "*")):
        with open(path, encoding="utf-8") as f:
            for m in pat.finditer(f.read()):
                seen.add(re.sub(r"\s+", " ", m.group(0)))
    assert seen, "no kernel names found under profiles/"
    unknown = sorted(seen - covered)
    assert not unknown, f"profiled kernels without a parity case: {unknown}"


def test_config_query_validates_like_the_entry_points():
    L = lib()
    import ctypes
    buf = ctypes.create_string_buffer(64)
    assert L.q4_linear_config(0, 4, 17, 64, 128, 128, 256, 256, buf, 64) == Q4_ERR_SHAPE     # m > 16 in a GEMV
    assert L.q4_linear_config(1, 4, 17, 64, 128, 128, 256, 256, buf, 64) == 0
    assert L.q4_linear_config(0, 4, 1, 64, 144, 48, 256, 256, buf, 64) == Q4_ERR_GROUP
    assert L.q4_linear_config(0, 4, 1, 64, 128, 256, 256, 256, buf, 64) == Q4_ERR_SHAPE     # n_in % g
    assert L.q4_linear_config(2, 4, 1, 64, 128, 128, 256, 256, buf, 64) == Q4_ERR_SHAPE     # op
    assert L.q4_linear_config(0, 5, 1, 64, 128, 128, 256, 256, buf, 64) == Q4_ERR_SHAPE     # bits
    assert L.q4_linear_config(0, 4, 1, 64, 128, 128, None, 256, buf, 64) == Q4_ERR_NULL
    assert L.q4_linear_config(0, 4, 1, 64, 128, 128, 256, 256, None, 64) == Q4_ERR_NULL
    small = ctypes.create_string_buffer(8)
    assert L.q4_linear_config(0, 4, 1, 64, 128, 128, 256, 256, small, 8) == 0
    assert len(small.value) == 7                       # truncated, NUL-terminated


def test_one_token_bench_calls_take_row_streaming():
    """The benchmark's m = 1 GEMVs (INT4 grouped, INT8 per-channel) run on the
    row-streaming kernels; a dispatch change that sent them back to the MFMA
    kernels would cost 12-31 % per launch."""
    calls = [c for c in bench_cases() if c.kind == "gemv" and c.m == 1 and c.n_in <= 16384]
    assert calls
    for c in calls:
        name = config(c)
        assert name.startswith("gemv_rowstream"), f"{c}: {name}"
