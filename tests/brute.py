"""Pure-Python brute-force checker for group-wise quantization results.

It does not recompute the quantizer's formula.  It states what a correct
result must be and checks that with exact rational arithmetic
(`fractions.Fraction` of the binary32 values):

  * the fp32 scale spans the group's range in 2^b - 1 steps (asymmetric) or
    maps max|w| to 2^(b-1) - 1 (symmetric), up to binary32 rounding;
  * the zero-point is the integer offset whose code 0 lands nearest the
    group minimum, clipped to the code range;
  * every code is a nearest grid point: over all 2^b codes, none lies closer
    to w than the chosen one (beyond the rounding of the fp32 division), and
    exact ties go to the even offset (round-half-to-even);
  * the codes read back from the packed words in natural order (32/b codes
    per word, element k at bits b*(k % (32/b))).
b is 4 or 8; a group may be a whole row (per-channel).
"""
from fractions import Fraction

import numpy as np

F32_ONE_E8 = Fraction(float(np.float32(1e-8)))
# Slack for the binary32 steps (the division w/s and the range arithmetic).
EPS = Fraction(1, 1 << 21)


def fr(v):
    return Fraction(float(v))


def unpack_codes(words_row, n_in, bits=4):
    """Codes of one row, element k from bits b(k % (32/b)).. of word k // (32/b)."""
    per = 32 // bits
    mask = (1 << bits) - 1
    return [(int(words_row[k // per]) >> (bits * (k % per))) & mask for k in range(n_in)]


def check_group(vals, s, z, codes, symmetric, where, bits=4):
    """Raise AssertionError describing the first violation in one group.

    vals: binary32 weights; s: binary32 scale before storage; z: integer
    zero-point (0..2^b-1 asymmetric, 2^(b-1) symmetric); codes: stored codes
    0..2^b-1.
    """
    top = (1 << bits) - 1             # asymmetric steps / top code
    half = 1 << (bits - 1)            # symmetric offset
    vals = [fr(v) for v in vals]
    S = fr(s)
    assert S > 0, f"{where}: scale {s} not positive"
    if symmetric:
        qmax = half - 1
        amax = max(abs(v) for v in vals)
        if amax / qmax > F32_ONE_E8 * (1 + EPS):
            assert abs(qmax * S - amax) <= amax * EPS, \
                f"{where}: {qmax}*s={qmax*float(S)} vs max|w|={float(amax)}"
        elif amax / qmax < F32_ONE_E8 * (1 - EPS):
            assert S == F32_ONE_E8, f"{where}: degenerate scale {s} != 1e-8"
        assert z == half, f"{where}: symmetric stored zero-point {z} != {half}"
        lo, hi = -half, half - 1
        offsets = [u - half for u in codes]
    else:
        mn, mx = min(vals), max(vals)
        rng = mx - mn
        if rng / top > F32_ONE_E8 * (1 + EPS):
            assert abs(top * S - rng) <= rng * EPS, f"{where}: {top}*s={top*float(S)} vs range={float(rng)}"
        elif rng / top < F32_ONE_E8 * (1 - EPS):
            assert S == F32_ONE_E8, f"{where}: degenerate scale {s} != 1e-8"
        t = -mn / S
        assert 0 <= z <= top, f"{where}: zero-point {z} outside [0, {top}]"
        if t < Fraction(-1, 2) - EPS * abs(t):
            assert z == 0, f"{where}: min above 0, zero-point {z} should clip to 0"
        elif t > Fraction(2 * top + 1, 2) + EPS * abs(t):
            assert z == top, f"{where}: max below 0, zero-point {z} should clip to {top}"
        else:
            best = min(range(top + 1), key=lambda c: abs(t - c))
            assert abs(t - z) <= abs(t - best) + EPS * abs(t) + EPS, \
                f"{where}: zero-point {z} not nearest to -min/s={float(t)}"
        lo, hi = -z, top - z
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


def check_matrix(w, packed, scales_f16_bits, zeros_f16_bits, s32, group_size, symmetric, bits=4):
    """Brute-force check of a whole (small) quantized matrix."""
    n_out, n_in = w.shape
    zeros = np.asarray(zeros_f16_bits, dtype=np.uint16).view(np.float16).astype(np.float32)
    want_scales = np.asarray(s32, dtype=np.float32).astype(np.float16).view(np.uint16)
    assert np.array_equal(np.asarray(scales_f16_bits), want_scales), "stored scales are not fp16(s)"
    for n in range(n_out):
        codes = unpack_codes(packed[n], n_in, bits)
        for j in range(n_in // group_size):
            z = float(zeros[n, j])
            assert z == int(z), f"row {n} group {j}: stored zero-point {z} not an integer"
            sl = slice(j * group_size, (j + 1) * group_size)
            check_group(w[n, sl], s32[n, j], int(z), codes[sl], symmetric,
                        f"row {n} group {j}", bits)
