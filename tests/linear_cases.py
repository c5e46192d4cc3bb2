"""Shapes of the linear-layer parity tests, kept in one place so that a CPU
test can check them against the library's kernel selection
(`q4_linear_config`) without a GPU.

Each case is (kind, bits, m, n_out, n_in, group_size, align): kind "gemv" or
"gemm", INT4 or INT8 weights, `align` the address modulo 512 at which the
scale and zero-point arrays start (the prefill kernel reads runs of groups
when they are 16- or 4-byte aligned).

COVERAGE holds one case per kernel configuration the dispatch rules can
reach: the cheapest shape that selects it, preferring ragged ones (a partial
last tile of 16 channels, a partial last 128-wide block, m not a power of
two).  bench_cases() gives the exact linear-layer shapes the benchmark times.
"""
from collections import namedtuple

Case = namedtuple("Case", "kind bits m n_out n_in group_size align")

COVERAGE = [Case(*c) for c in (
    ("gemm", 4, 17, 17, 32, 32, 256),          # gemm_kernel<256, 128, 4, false, 1>
    ("gemm", 4, 17, 17, 96, 96, 256),          # gemm_kernel<256, 128, 4, true, 1>
    ("gemm", 4, 17, 17, 128, 64, 256),         # gemm_kernel<256, 128, 4, true, 2>
    ("gemm", 4, 17, 17, 1024, 64, 256),        # gemm_kernel<256, 128, 4, true, 8>
    ("gemm", 8, 17, 17, 32, 32, 256),          # gemm_kernel<256, 128, 8, true, 1>
    ("gemm", 8, 17, 17, 128, 64, 256),         # gemm_kernel<256, 128, 8, true, 2>
    ("gemm", 8, 17, 17, 1024, 64, 256),        # gemm_kernel<256, 128, 8, true, 8>
    ("gemm", 4, 300, 100, 1024, 128, 260),     # 4-byte aligned metadata: runs of 2
    ("gemm", 8, 300, 100, 2048, 128, 258),     # 2-byte aligned metadata: per-step gathers
    ("gemv", 4, 2, 17, 2016, 32, 256),         # gemv_resident_kernel<16, 1, 1, 4, false, 4, false>
    ("gemv", 4, 1, 8192, 16416, 32, 256),      # gemv_resident_kernel<16, 1, 2, 1, false, 4, true>
    ("gemv", 4, 2, 17, 32, 32, 256),           # gemv_resident_kernel<4, 1, 1, 2, false, 4, false>
    ("gemv", 8, 2, 17, 32, 32, 256),           # gemv_resident_kernel<4, 1, 1, 2, false, 8, false>
    ("gemv", 8, 1, 4112, 2016, 32, 256),       # gemv_resident_kernel<4, 1, 1, 2, false, 8, true>
    ("gemv", 4, 2, 17, 128, 128, 256),         # gemv_resident_kernel<4, 1, 1, 2, true, 4, false>
    ("gemv", 8, 1, 12304, 2016, 32, 256),      # gemv_resident_kernel<4, 2, 1, 1, false, 8, true>
    ("gemv", 4, 1, 12304, 2016, 32, 256),      # gemv_resident_kernel<4, 2, 1, 2, false, 4, false>
    ("gemv", 4, 1, 12304, 2048, 128, 256),     # gemv_resident_kernel<4, 2, 1, 2, true, 4, false>
    ("gemv", 4, 1, 12304, 8192, 128, 256),     # gemv_resident_kernel<4, 2, 2, 2, true, 4, true>
    ("gemv", 4, 1, 17, 2016, 32, 256),         # gemv_resident_kernel<8, 1, 1, 2, false, 4, false>
    ("gemv", 8, 2, 17, 2016, 32, 256),         # gemv_resident_kernel<8, 1, 1, 2, false, 8, false>
    ("gemv", 8, 1, 17, 2016, 32, 256),         # gemv_resident_kernel<8, 1, 1, 2, false, 8, true>
    ("gemv", 4, 2, 17, 2048, 128, 256),        # gemv_resident_kernel<8, 1, 1, 2, true, 4, false>
    ("gemv", 4, 1, 17, 16416, 32, 256),        # gemv_resident_kernel<8, 1, 1, 3, false, 4, false>
    ("gemv", 8, 1, 17, 16416, 32, 256),        # gemv_resident_kernel<8, 1, 1, 3, false, 8, true>
    ("gemv", 4, 1, 17, 8192, 128, 256),        # gemv_resident_kernel<8, 1, 1, 3, true, 4, false>
    ("gemv", 4, 1, 8192, 16384, 128, 256),     # gemv_resident_kernel<8, 1, 2, 2, true, 4, true>
    ("gemv", 8, 5, 17, 2016, 32, 256),         # gemv_resident_kernel<8, 2, 1, 2, false, 8, true>
    ("gemv", 4, 2, 4096, 2048, 128, 256),      # gemv_resident_kernel<8, 2, 1, 2, true, 4, false>
    ("gemv", 8, 5, 10240, 2016, 32, 256),      # gemv_resident_kernel<8, 4, 1, 1, false, 8, true>
    ("gemv", 4, 2, 10240, 2048, 128, 256),     # gemv_resident_kernel<8, 4, 2, 1, true, 4, true>
    ("gemv", 4, 4, 17, 16416, 32, 256),        # gemv_window_kernel<16, 2, 1, false, 8, 4>
    ("gemv", 8, 4, 17, 16416, 32, 256),        # gemv_window_kernel<16, 2, 1, false, 8, 8>
    ("gemv", 4, 5, 17, 16384, 128, 256),       # gemv_window_kernel<16, 2, 1, true, 8, 4>
    ("gemv", 4, 9, 17, 16416, 32, 256),        # gemv_window_kernel<8, 2, 1, false, 16, 4>
    ("gemv", 8, 9, 17, 16416, 32, 256),        # gemv_window_kernel<8, 2, 1, false, 16, 8>
    ("gemv", 4, 10, 17, 8192, 128, 256),       # gemv_window_kernel<8, 2, 1, true, 16, 4>
)]


def bench_cases():
    """The benchmark's timed linear-layer calls (bench.timed_linear_calls),
    which tests/test_gpu_bench_shapes.py runs on the benchmark's own inputs."""
    import bench
    return sorted({Case(c.kind, c.bits, c.m, c.n_out, c.n_in, c.group_size, 256)
                   for c in bench.timed_linear_calls()})
