"""Seeded random linear-layer shapes through q4_gemv / q8_gemv and q4_gemm
against the oracle: INT4 and INT8, m from 1 to 16 (and prefill sizes for the
GEMM), every group size and per-channel groups, ragged row counts and row
lengths, and scale / zero-point arrays at 16-, 4- and 2-byte alignment.  Each
case is checked like the dispatch-coverage cases (packed codes bit for bit on
the checked rows, y within |y - y_ref| <= 2e-3 sum|x w'| + 1e-5)."""
import numpy as np
import pytest

from linear_cases import Case
from test_gpu_dispatch_coverage import run_case

pytestmark = pytest.mark.gpu


def random_cases(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        bits = int(rng.choice([4, 8]))
        g = int(rng.choice([32, 64, 128, 256, 0]))
        kind = "gemm" if rng.random() < 0.2 else "gemv"
        if g:
            n_in = g * int(rng.integers(1, max(2, 16416 // g)))
        else:
            n_in = 32 * int(rng.integers(1, 513))
        g = g or n_in
        if kind == "gemv":
            m = int(rng.choice([1, 1, 1, 2, 3, 4, 5, 8, 8, 11, 16]))
            n_out = int(rng.integers(1, 5000))
            if rng.random() < 0.1:
                n_out = int(rng.integers(32768, 40000))
                n_in = min(n_in, 4096 - 4096 % g) or g
        else:
            m = int(rng.integers(17, 600))
            n_out = int(rng.integers(1, 1200))
            n_in = min(n_in, 4096 - 4096 % g) or g
        align = int(rng.choice([256, 260, 258]))
        out.append(Case(kind, bits, m, n_out, n_in, g, align))
    return out


CASES = random_cases(40, 2026)


def case_id(c):
    return f"{c.kind}-int{c.bits}-m{c.m}-{c.n_out}x{c.n_in}-g{c.group_size}-a{c.align % 16}"


@pytest.mark.parametrize("case", CASES, ids=case_id)
def test_random_shape(orc, case):
    run_case(orc, case, seed=case.n_out * 7 + case.n_in + case.m)
