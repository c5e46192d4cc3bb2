"""Pure-Python brute-force checker for group-wise quantization results.

It does not recompute the quantizer's formula.  It states what a correct
result must be and checks that with exact rational arithmetic
(`fractions.Fraction` of the binary32 values):

  * the fp32 scale spans the group's range in 2^b - 1 steps (asymmetric) or
    maps max|w| to 2^(b-1) - 1 (symmetric), up to binary32 rounding;
  * the zero-point is the integer offset whose code 0 lands nearest the
    group minimum, clipped to the code range;
  * every code is a nearest grid point: over all 16 codes, none lies closer
    to w than the chosen one (beyond the rounding of the fp32 division), and
    exact ties go to the even offset (round-half-to-even);
  * the codes read back from the packed words in natural nibble order.
"""
from fractions import Fraction

import numpy as np

F32_ONE_E8 = Fraction(float(np.float32(1e-8)))
# Slack for the binary32 steps (the division w/s and the range arithmetic).
EPS = Fraction(1, 1 << 21)


def fr(v):
    return Fraction(float(v))


def unpack_codes(words_row, n_in):
    """Codes of one row, element k from bits 4(k%8).. of word k//8."""
    return [(int(words_row[k // 8]) >> (4 * (k % 8))) & 0xF for k in range(n_in)]


def check_group(vals, s, z, codes, symmetric, where):
    """Raise AssertionError describing the first violation in one group.

    vals: binary32 weights; s: binary32 scale before storage; z: integer
    zero-point (0..15 asymmetric, 8 symmetric); codes: stored nibbles 0..15.
    """
    vals = [fr(v) for v in vals]
    S = fr(s)
    assert S > 0, f"{where}: scale {s} not positive"
    if symmetric:
        amax = max(abs(v) for v in vals)
        if amax / 7 > F32_ONE_E8 * (1 + EPS):
            assert abs(7 * S - amax) <= amax * EPS, f"{where}: 7*s={7*float(S)} vs max|w|={float(amax)}"
        elif amax / 7 < F32_ONE_E8 * (1 - EPS):
            assert S == F32_ONE_E8, f"{where}: degenerate scale {s} != 1e-8"
        assert z == 8, f"{where}: symmetric stored zero-point {z} != 8"
        lo, hi = -8, 7
        offsets = [u - 8 for u in codes]
    else:
        mn, mx = min(vals), max(vals)
        rng = mx - mn
        if rng / 15 > F32_ONE_E8 * (1 + EPS):
            assert abs(15 * S - rng) <= rng * EPS, f"{where}: 15*s={15*float(S)} vs range={float(rng)}"
        elif rng / 15 < F32_ONE_E8 * (1 - EPS):
            assert S == F32_ONE_E8, f"{where}: degenerate scale {s} != 1e-8"
        t = -mn / S
        assert 0 <= z <= 15, f"{where}: zero-point {z} outside [0, 15]"
        if t < Fraction(-1, 2) - EPS * abs(t):
            assert z == 0, f"{where}: min above 0, zero-point {z} should clip to 0"
        elif t > Fraction(31, 2) + EPS * abs(t):
            assert z == 15, f"{where}: max below 0, zero-point {z} should clip to 15"
        else:
            best = min(range(16), key=lambda c: abs(t - c))
            assert abs(t - z) <= abs(t - best) + EPS * abs(t) + EPS, \
                f"{where}: zero-point {z} not nearest to -min/s={float(t)}"
        lo, hi = -z, 15 - z
        offsets = [u - z for u in codes]

    for i, (v, c) in enumerate(zip(vals, offsets)):
        tw = v / S
        slack = EPS * (abs(tw) + 1)
        if lo < c < hi:
            # enumerate every representable code: none may be clearly closer
            for cand in range(lo, hi + 1):
                assert abs(tw - c) <= abs(tw - cand) + slack, \
                    f"{where}[{i}]: code offset {c} but {cand} is nearer to w/s={float(tw)}"
            if tw.denominator == 2 and abs(tw) < (1 << 22):
                assert c % 2 == 0, f"{where}[{i}]: tie w/s={float(tw)} must round to even, got {c}"
        elif c == hi:
            assert tw >= hi - Fraction(1, 2) - slack, f"{where}[{i}]: top code for w/s={float(tw)}"
        elif c == lo:
            assert tw <= lo + Fraction(1, 2) + slack, f"{where}[{i}]: bottom code for w/s={float(tw)}"
        else:
            raise AssertionError(f"{where}[{i}]: offset {c} outside [{lo}, {hi}]")


def check_matrix(w, packed, scales_f16_bits, zeros_f16_bits, s32, group_size, symmetric):
    """Brute-force check of a whole (small) quantized matrix."""
    n_out, n_in = w.shape
    zeros = np.asarray(zeros_f16_bits, dtype=np.uint16).view(np.float16).astype(np.float32)
    want_scales = np.asarray(s32, dtype=np.float32).astype(np.float16).view(np.uint16)
    assert np.array_equal(np.asarray(scales_f16_bits), want_scales), "stored scales are not fp16(s)"
    for n in range(n_out):
        codes = unpack_codes(packed[n], n_in)
        for j in range(n_in // group_size):
            z = float(zeros[n, j])
            assert z == int(z), f"row {n} group {j}: stored zero-point {z} not an integer"
            sl = slice(j * group_size, (j + 1) * group_size)
            check_group(w[n, sl], s32[n, j], int(z), codes[sl], symmetric,
                        f"row {n} group {j}")
