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
    ("gemm", 4, 300, 100, 1024, 128, 260),     # gemm_kernel<256, 128, 4, true, 2> (4-byte aligned metadata: runs of 2)
    ("gemm", 4, 17, 17, 1024, 64, 256),        # gemm_kernel<256, 128, 4, true, 8>
    ("gemm", 8, 17, 17, 32, 32, 256),          # gemm_kernel<256, 128, 8, true, 1>
    ("gemm", 8, 300, 100, 2048, 128, 258),     # gemm_kernel<256, 128, 8, true, 1> (2-byte aligned metadata: per-step gathers)
    ("gemm", 8, 17, 17, 128, 64, 256),         # gemm_kernel<256, 128, 8, true, 2>
    ("gemm", 8, 17, 17, 1024, 64, 256),        # gemm_kernel<256, 128, 8, true, 8>
    ("gemv", 4, 3, 32777, 2048, 128, 256),     # gemv_persistent_kernel<8, 4, 2, 1, true, true> (ragged last group)
    ("gemv", 4, 8, 32800, 4096, 256, 256),     # gemv_persistent_kernel<8, 4, 2, 1, true, true> (groups of 256)
    ("gemv", 4, 2, 17, 2016, 32, 256),         # gemv_resident_kernel<16, 1, 1, 4, false, 4, false>
    ("gemv", 4, 1, 8192, 16416, 32, 256),      # gemv_resident_kernel<16, 1, 2, 1, false, 4, true>
    ("gemv", 4, 2, 17, 32, 32, 256),           # gemv_resident_kernel<4, 1, 1, 2, false, 4, false>
    ("gemv", 8, 2, 17, 32, 32, 256),           # gemv_resident_kernel<4, 1, 1, 2, false, 8, false>
    ("gemv", 8, 1, 4112, 2016, 32, 258),       # gemv_resident_kernel<4, 1, 1, 2, false, 8, true> (2-byte aligned metadata)
    ("gemv", 4, 2, 17, 128, 128, 256),         # gemv_resident_kernel<4, 1, 1, 2, true, 4, false>
    ("gemv", 8, 1, 12304, 2016, 32, 258),      # gemv_resident_kernel<4, 2, 1, 1, false, 8, true> (2-byte aligned metadata)
    ("gemv", 4, 1, 12304, 2016, 32, 258),      # gemv_resident_kernel<4, 2, 1, 2, false, 4, false> (2-byte aligned metadata)
    ("gemv", 4, 1, 12304, 2048, 128, 258),     # gemv_resident_kernel<4, 2, 1, 2, true, 4, false> (2-byte aligned metadata)
    ("gemv", 4, 1, 12304, 8192, 128, 258),     # gemv_resident_kernel<4, 2, 2, 2, true, 4, true> (2-byte aligned metadata)
    ("gemv", 4, 1, 17, 2016, 32, 258),         # gemv_resident_kernel<8, 1, 1, 2, false, 4, false> (2-byte aligned metadata: no row-streaming kernel)
    ("gemv", 8, 2, 17, 2016, 32, 256),         # gemv_resident_kernel<8, 1, 1, 2, false, 8, false>
    ("gemv", 8, 1, 17, 2016, 32, 258),         # gemv_resident_kernel<8, 1, 1, 2, false, 8, true> (2-byte aligned metadata)
    ("gemv", 4, 2, 17, 2048, 128, 256),        # gemv_resident_kernel<8, 1, 1, 2, true, 4, false>
    ("gemv", 4, 1, 17, 16416, 32, 256),        # gemv_resident_kernel<8, 1, 1, 3, false, 4, false>
    ("gemv", 8, 1, 17, 16416, 32, 256),        # gemv_resident_kernel<8, 1, 1, 3, false, 8, true>
    ("gemv", 4, 1, 17, 28672, 128, 256),       # gemv_resident_kernel<8, 1, 1, 3, true, 4, false>
    ("gemv", 8, 5, 17, 2016, 32, 256),         # gemv_resident_kernel<8, 2, 1, 2, false, 8, true>
    ("gemv", 4, 2, 4096, 2048, 128, 256),      # gemv_resident_kernel<8, 2, 1, 2, true, 4, false>
    ("gemv", 8, 5, 10240, 2016, 32, 256),      # gemv_resident_kernel<8, 4, 1, 1, false, 8, true>
    ("gemv", 4, 2, 10240, 2048, 128, 256),     # gemv_resident_kernel<8, 4, 2, 1, true, 4, true>
    ("gemv", 8, 1, 9, 64, 64, 256),            # gemv_rowstream8_kernel<1, 8> (per-channel, 64-code rows)
    ("gemv", 8, 1, 17, 32, 32, 256),           # gemv_rowstream8_kernel<1, 8>
    ("gemv", 8, 1, 17, 13312, 256, 256),       # gemv_rowstream8_kernel<13, 8>
    ("gemv", 8, 1, 1003, 16384, 16384, 256),   # gemv_rowstream8_kernel<16, 8> (per-channel, ragged rows)
    ("gemv", 8, 1, 17, 2016, 32, 256),         # gemv_rowstream8_kernel<2, 8>
    ("gemv", 8, 1, 4112, 2016, 32, 256),       # gemv_rowstream8_kernel<2, 8>
    ("gemv", 8, 1, 12304, 2016, 32, 256),      # gemv_rowstream8_kernel<2, 8>
    ("gemv", 8, 1, 17, 2080, 32, 256),         # gemv_rowstream8_kernel<3, 8>
    ("gemv", 8, 1, 1003, 4096, 4096, 260),     # gemv_rowstream8_kernel<4, 8> (per-channel, 4-byte aligned metadata)
    ("gemv", 8, 1, 17, 4224, 64, 256),         # gemv_rowstream8_kernel<5, 8>
    ("gemv", 8, 1, 17, 8192, 128, 256),        # gemv_rowstream8_kernel<8, 8>
    ("gemv", 8, 1, 17, 8320, 32, 256),         # gemv_rowstream8_kernel<9, 8>
    ("gemv", 8, 1, 517, 8320, 8320, 256),      # gemv_rowstream8_kernel<9, 8> (per-channel, n_in not a power of two)
    ("gemv", 4, 1, 9, 64, 32, 256),            # gemv_rowstream_kernel<1, 1, 8> (two-lane rows)
    ("gemv", 4, 1, 17, 2016, 2016, 256),       # gemv_rowstream_kernel<1, 1, 8> (per-channel)
    ("gemv", 4, 1, 17, 2016, 32, 256),         # gemv_rowstream_kernel<1, 1, 8>
    ("gemv", 4, 1, 17, 32, 32, 256),           # gemv_rowstream_kernel<1, 1, 8> (one 32-code row)
    ("gemv", 4, 1, 12304, 2016, 2016, 256),    # gemv_rowstream_kernel<1, 1, 8> (per-channel)
    ("gemv", 4, 1, 12304, 2016, 32, 256),      # gemv_rowstream_kernel<1, 1, 8>
    ("gemv", 4, 1, 12304, 2048, 128, 256),     # gemv_rowstream_kernel<1, 1, 8>
    ("gemv", 4, 1, 17, 4224, 32, 256),         # gemv_rowstream_kernel<3, 1, 8>
    ("gemv", 4, 1, 4101, 6144, 256, 256),      # gemv_rowstream_kernel<3, 1, 8> (groups of 256, ragged rows)
    ("gemv", 4, 1, 4101, 6144, 128, 260),      # gemv_rowstream_kernel<3, 1, 8> (4-byte aligned metadata)
    ("gemv", 4, 1, 17, 8192, 128, 256),        # gemv_rowstream_kernel<4, 1, 8>
    ("gemv", 4, 1, 12304, 8192, 128, 256),     # gemv_rowstream_kernel<4, 1, 8>
    ("gemv", 4, 1, 17, 8320, 32, 256),         # gemv_rowstream_kernel<5, 1, 8>
    ("gemv", 4, 1, 12301, 8320, 128, 256),     # gemv_rowstream_kernel<5, 1, 8> (ragged rows, odd group count, partial chunk)
    ("gemv", 4, 1, 1000, 13312, 32, 256),      # gemv_rowstream_kernel<7, 1, 8> (partial last chunk of 2048)
    ("gemv", 4, 1, 8192, 16384, 128, 256),     # gemv_rowstream_kernel<8, 1, 8>
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
