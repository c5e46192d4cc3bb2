"""Pins of the CPU oracle to facts that do not come from the oracle itself.

Each pin takes an `oracle.Oracle` and raises AssertionError when the oracle
disagrees with what the pages or the mathematics fix.  The same pins run
against deliberately broken copies of the oracle (tests/test_oracle_mutants.py)
to show that a plausible mistake anywhere in it is caught.
"""
import json
import os

import numpy as np
import torch

from brute import check_group, check_matrix
from w4a16_dequant_gemv_amd import synthetic

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name), encoding="utf-8") as f:
        return json.load(f)


def _f16_bits_to_f32(h):
    return np.asarray(h, dtype=np.uint16).view(np.float16).astype(np.float32)


def _f16_bits(a_f32):
    """fp16 bit patterns by torch's CPU conversion (hardware F16C, IEEE RNE)."""
    t = torch.from_numpy(np.ascontiguousarray(a_f32, dtype=np.float32)).half()
    return t.view(torch.int16).numpy().view(np.uint16)


# ---------------------------------------------------------------------------
# Worked example: the interview guide's §3, per-tensor symmetric INT8.
# ---------------------------------------------------------------------------
def pin_worked_example(orc, quick=False):
    g = _golden("worked_example.json")
    rng = np.random.default_rng(11)
    x = rng.uniform(-3, 3, size=4096).astype(np.float32)       # normal channels
    x[17] = g["max_abs"]                                         # the outlier channel
    x[901] = -63.0
    x[5] = g["x"]
    s, z, q = orc.quantize_group(x, bits=g["bits"], symmetric=g["symmetric"])
    tol = 0.5 * 10.0 ** (-g["scale_printed_digits"])
    assert abs(float(s) - g["scale_printed"]) <= tol, f"scale {s} vs printed {g['scale_printed']}"
    assert z == 0
    assert int(q[5]) == g["q"], f"q(0.5) = {q[5]}"
    assert int(q[17]) == 2 ** (g["bits"] - 1) - 1, "max|x| must map to the top code"
    x_hat = float(s) * (int(q[5]) - z)
    assert abs(x_hat - g["x_hat_printed"]) <= tol, f"x_hat {x_hat}"
    rel = abs(x_hat - g["x"]) / g["x"] * 100
    assert round(rel) == g["rel_error_percent_printed"], f"error {rel}%"
    # small channels are crushed onto few codes, as the page describes
    assert set(np.unique(q[np.abs(x) < 1.0])) <= {-1, 0, 1}


# ---------------------------------------------------------------------------
# Brute force over every code on 2x256 matrices.
# ---------------------------------------------------------------------------
def _small_cases():
    cases = []
    w = synthetic.normal_weight(2, 256, seed=21, std=0.02, n_outlier_cols=3)
    cases.append(w)
    cases.append(synthetic.student_t_weight(2, 256, seed=22, group_size=32,
                                            const_frac=0.0, zero_frac=0.0))
    rng = np.random.default_rng(23)
    u = rng.uniform(-1, 1, size=(2, 256)).astype(np.float32)
    u[0, :128] = np.abs(u[0, :128]) + 0.25          # all-positive groups
    u[1, 128:] = -np.abs(u[1, 128:]) - 0.25         # all-negative groups
    cases.append(u)
    return cases


def pin_brute_force(orc, quick=False):
    for ci, w in enumerate(_small_cases()):
        for g in (32, 128):
            for sym in (False, True):
                packed, scales, zeros, s32 = orc.quantize_pack(w, g, sym)
                try:
                    check_matrix(w, packed, scales, zeros, s32, g, sym)
                except AssertionError as e:
                    raise AssertionError(f"case {ci} g={g} sym={sym}: {e}") from None


# ---------------------------------------------------------------------------
# Exact ties round to even (the pages round with torch.round / np.round).
# ---------------------------------------------------------------------------
def pin_ties_to_even(orc, quick=False):
    # range [-7, 8] gives s = 1 exactly and z = 7; w/s is then w itself
    vals = [-7.0, 8.0, 0.5, 1.5, 2.5, -0.5, -1.5, 3.5, -2.5, 4.5] + [0.0] * 22
    w = np.array([vals], dtype=np.float32)
    packed, scales, zeros, s32 = orc.quantize_pack(w, 32, False)
    assert float(s32[0, 0]) == 1.0 and float(_f16_bits_to_f32(zeros)[0, 0]) == 7.0
    codes = [(int(packed[0, k // 8]) >> (4 * (k % 8))) & 0xF for k in range(32)]
    want = [round(v) + 7 for v in vals]             # Python's round: half to even
    assert codes == want, f"tie codes {codes[:10]} != {want[:10]}"
    # symmetric: max|w| = 7 gives s = 1, ties on the signed codes
    vals_s = [7.0, -6.5, 0.5, 1.5, 2.5, -0.5, -3.5, 5.5] + [0.0] * 24
    w = np.array([vals_s], dtype=np.float32)
    packed, scales, zeros, s32 = orc.quantize_pack(w, 32, True)
    assert float(s32[0, 0]) == 1.0
    codes = [(int(packed[0, k // 8]) >> (4 * (k % 8))) & 0xF for k in range(32)]
    assert codes == [round(v) + 8 for v in vals_s], f"symmetric tie codes {codes[:8]}"


# ---------------------------------------------------------------------------
# Zero-point clipping to [0, 15] for one-signed groups.
# ---------------------------------------------------------------------------
def pin_zero_clip(orc, quick=False):
    w = np.empty((2, 32), dtype=np.float32)
    w[0] = np.linspace(0.5, 2.0, 32)
    w[1] = np.linspace(-2.0, -0.5, 32)
    packed, scales, zeros, s32 = orc.quantize_pack(w, 32, False)
    z = _f16_bits_to_f32(zeros)[:, 0]
    assert z[0] == 0.0, f"all-positive group: zero-point {z[0]} should clip to 0"
    assert z[1] == 15.0, f"all-negative group: zero-point {z[1]} should clip to 15"


# ---------------------------------------------------------------------------
# Reconstruction bound |w - w'| <= s/2 (+ fp16 storage slack).
# ---------------------------------------------------------------------------
def _bound_cases(quick):
    rows = 32 if quick else 128
    return [
        ("normal+outliers", synthetic.normal_weight(rows, 4096, seed=31, std=0.02,
                                                    n_outlier_cols=8)),
        ("student-t", synthetic.student_t_weight(rows, 2048, seed=32, group_size=128,
                                                 const_frac=0.0, zero_frac=0.0)),
    ]


def pin_reconstruction_bound(orc, quick=False):
    for name, w in _bound_cases(quick):
        for g in (32, 128):
            for sym in (False, True):
                packed, scales, zeros, s32 = orc.quantize_pack(w, g, sym)
                wd = orc.dequant(packed, scales, zeros, g)
                n_out, n_in = w.shape
                G = n_in // g
                s = s32.astype(np.float64).repeat(g, axis=1)
                sh = _f16_bits_to_f32(scales).astype(np.float64).repeat(g, axis=1)
                grp = w.reshape(n_out, G, g)
                if sym:
                    ok = (np.abs(grp).max(axis=2) / 7 > 1e-7)
                    cmax = 8
                else:
                    mn, mx = grp.min(axis=2), grp.max(axis=2)
                    ok = (mn <= 0) & (mx >= 0) & ((mx - mn) / 15 > 1e-7)
                    cmax = 15
                ok = ok.repeat(g, axis=1)
                err = np.abs(w.astype(np.float64) - wd.astype(np.float64))
                bound = s * (0.5 + 2.0 ** -18) + cmax * np.abs(s - sh)
                bad = ok & (err > bound)
                assert not bad.any(), (f"{name} g={g} sym={sym}: |w-w'| exceeds s/2 at "
                                       f"{np.argwhere(bad)[:3].tolist()}")
                assert np.isfinite(wd).all()


# ---------------------------------------------------------------------------
# Quantize o dequantize o quantize == quantize.
# ---------------------------------------------------------------------------
def _codes(packed):
    shifts = (4 * np.arange(8, dtype=np.uint32))
    return ((packed[..., None] >> shifts) & 0xF).reshape(packed.shape[0], -1)


def pin_idempotence(orc, quick=False):
    for name, w in _bound_cases(quick):
        for g in (32, 128):
            for sym in (False, True):
                p1, s1, z1, _ = orc.quantize_pack(w, g, sym)
                wd = orc.dequant(p1, s1, z1, g)
                p2, s2, z2, _ = orc.quantize_pack(wd, g, sym)
                n_out, n_in = w.shape
                G = n_in // g
                c1 = _codes(p1).reshape(n_out, G, g)
                c2 = _codes(p2).reshape(n_out, G, g)
                sh = _f16_bits_to_f32(s1)
                if sym:
                    sel = sh > 0
                else:
                    sel = (c1.min(axis=2) == 0) & (c1.max(axis=2) == 15) & (sh > 0)
                assert sel.mean() > 0.5, f"{name} g={g}: too few qualifying groups"
                same = (c1 == c2).all(axis=2) & (s1 == s2) & (z1 == z2)
                bad = sel & ~same
                assert not bad.any(), (f"{name} g={g} sym={sym}: Q(D(Q(W))) != Q(W) in "
                                       f"{int(bad.sum())} groups, first {np.argwhere(bad)[0].tolist()}")


# ---------------------------------------------------------------------------
# Groups that lie exactly on a grid come back exactly.
# ---------------------------------------------------------------------------
def pin_grid_exact(orc, quick=False):
    rng = np.random.default_rng(41)
    g, rows = 128, 16
    w = np.empty((rows, 4 * g), dtype=np.float32)
    expect = []
    for r in range(rows):
        for j in range(4):
            s = np.float32(np.float16(rng.uniform(1e-3, 0.2)))       # fp16-exact scale
            z = int(rng.integers(0, 16))
            u = rng.integers(0, 16, size=g)
            u[rng.integers(0, g)] = 0
            u[rng.integers(0, g)] = 15
            w[r, j * g:(j + 1) * g] = s * (u - z).astype(np.float32)
            expect.append((r, j, s, z, u))
    packed, scales, zeros, s32 = orc.quantize_pack(w, g, False)
    codes = _codes(packed).reshape(rows, 4, g)
    sh = _f16_bits_to_f32(scales)
    zh = _f16_bits_to_f32(zeros)
    for r, j, s, z, u in expect:
        assert sh[r, j] == s, f"row {r} group {j}: scale {sh[r, j]} != {s}"
        assert zh[r, j] == z, f"row {r} group {j}: zero {zh[r, j]} != {z}"
        assert np.array_equal(codes[r, j], u), f"row {r} group {j}: codes differ"
    wd = orc.dequant(packed, scales, zeros, g)
    assert np.array_equal(wd.view(np.uint32), w.view(np.uint32)), "grid-exact W not reproduced bitwise"


# ---------------------------------------------------------------------------
# Constant groups (max == min): no NaN or Inf, closed-form codes.
# ---------------------------------------------------------------------------
def pin_constant_groups(orc, quick=False):
    g = 32
    consts = [0.75, -0.75, 0.0, -0.0, 3e-9, 2e-8]
    w = np.repeat(np.array(consts, dtype=np.float32)[:, None], g, axis=1)
    packed, scales, zeros, s32 = orc.quantize_pack(w, g, False)
    codes = _codes(packed)
    sh = _f16_bits_to_f32(scales)[:, 0]
    zh = _f16_bits_to_f32(zeros)[:, 0]
    # s floors at 1e-8 (which rounds to fp16 zero); then w/s decides the code:
    # c = 0.75 -> 15 with z 0; c = -0.75 -> 0 with z 15; c = +-0 -> 0 with z 0;
    # c = 3e-9 -> rint(0.3) = 0; c = 2e-8 -> rint(2) = 2 with z 0.
    assert np.all(s32[:, 0] == np.float32(1e-8)) and np.all(sh == 0.0)
    want = [(15, 0), (0, 15), (0, 0), (0, 0), (0, 0), (2, 0)]
    for i, (u, z) in enumerate(want):
        assert np.all(codes[i] == u) and zh[i] == z, f"constant {consts[i]}: codes {codes[i][0]}, z {zh[i]}"
    wd = orc.dequant(packed, scales, zeros, g)
    assert np.all(wd == 0.0) and np.isfinite(wd).all()
    # symmetric: a nonzero constant is reconstructed through s = |c|/7
    packed, scales, zeros, s32 = orc.quantize_pack(w, g, True)
    codes = _codes(packed)
    assert np.all(codes[0] == 15) and np.all(codes[1] == 1) and np.all(codes[2] == 8)
    wd = orc.dequant(packed, scales, zeros, g)
    assert abs(wd[0, 0] - 0.75) < 1e-3 and abs(wd[1, 0] + 0.75) < 1e-3 and wd[2, 0] == 0.0
    assert np.isfinite(wd).all()


# ---------------------------------------------------------------------------
# Storage accounting: 4.25 bits per weight at g=128, metadata shares.
# ---------------------------------------------------------------------------
def pin_storage_accounting(orc, quick=False):
    entries = _golden("storage_accounting.json")["entries"]
    w = synthetic.normal_weight(8, 4096, seed=51)
    for e in entries:
        if "effective_bits_printed" in e:
            g = e["group_size"]
            packed, scales, zeros, _ = orc.quantize_pack(w, g, False)
            assert scales.shape[1] == e["scales_per_output_channel_printed"]
            bits = 8 * (packed.nbytes + scales.nbytes + zeros.nbytes) / w.size
            assert abs(bits - e["effective_bits_printed"]) < 1e-9, f"{bits} bits/weight"
        if "metadata_percent_printed" in e:
            g = e["group_size"]
            packed, scales, zeros, _ = orc.quantize_pack(w, g, False)
            share = 100.0 * scales.nbytes / packed.nbytes
            assert abs(share - e["metadata_percent_printed"]) < 0.05 + 1e-9, f"{share}%"
        if "int4_gb_printed" in e:
            packed, _, _, _ = orc.quantize_pack(w, 128, False)
            gb = e["params"] * (packed.nbytes / w.size) / 1e9
            assert gb == e["int4_gb_printed"]


# ---------------------------------------------------------------------------
# binary32 -> binary16 against torch's hardware conversion, every pattern.
# ---------------------------------------------------------------------------
def pin_f16_converter(orc, quick=False):
    chunk = 1 << 26
    if quick:
        rng = np.random.default_rng(61)
        starts = [int(x) << 20 for x in rng.choice(1 << 12, size=16, replace=False)]
        starts += [0x33000000, 0x387FF000, 0x477FE000, 0x7F7FF000]
        count = 1 << 16
    else:
        starts = list(range(0, 1 << 32, chunk))
        count = chunk
    for first in starts:
        bits = np.arange(first, first + count, dtype=np.uint64).astype(np.uint32)
        f = bits.view(np.float32)
        got = orc.f32_bits_range_to_f16(first, count)
        want = _f16_bits(f)
        nan = np.isnan(f)
        bad = (got != want) & ~nan
        assert not bad.any(), (f"fp32 {hex(int(bits[bad][0]))}: {hex(int(got[bad][0]))} "
                               f"vs {hex(int(want[bad][0]))}")
        gh = got[nan]
        assert np.all(((gh & 0x7C00) == 0x7C00) & ((gh & 0x3FF) != 0)), "NaN must stay NaN"
    # widening: every half pattern, exact
    h = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = orc.f16_to_f32(h)
    want = h.view(np.float16).astype(np.float32)
    nan = np.isnan(want)
    assert np.array_equal(got.view(np.uint32)[~nan], want.view(np.uint32)[~nan])
    assert np.isnan(got[nan]).all()


# ---------------------------------------------------------------------------
# Dequantization against an independent unpack with numpy's fp16.
# ---------------------------------------------------------------------------
def pin_dequant(orc, quick=False):
    rng = np.random.default_rng(71)
    n_out, n_in, g = 24, 512, 64
    packed = rng.integers(0, 1 << 32, size=(n_out, n_in // 8), dtype=np.uint64).astype(np.uint32)
    s = rng.uniform(0, 0.1, size=(n_out, n_in // g)).astype(np.float16)
    s[0, 0] = 0.0
    s[1, 1] = np.float16(6e-8)                    # fp16 subnormal
    z = rng.integers(0, 16, size=(n_out, n_in // g)).astype(np.float16)
    got = orc.dequant(packed, s.view(np.uint16), z.view(np.uint16), g)
    codes = _codes(packed).astype(np.int64)
    want = (s.astype(np.float32).repeat(g, axis=1)
            * (codes - z.astype(np.int64).repeat(g, axis=1)).astype(np.float32))
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), "dequant differs bitwise"


# ---------------------------------------------------------------------------
# Reference product against a numpy float64 matmul, one-hot and zero inputs.
# ---------------------------------------------------------------------------
def pin_linear_ref(orc, quick=False):
    rng = np.random.default_rng(81)
    m, n_out, n_in = 5, 96, 1024
    x = rng.standard_normal((m, n_in)).astype(np.float16)
    wd = (rng.standard_normal((n_out, n_in)) * 0.02).astype(np.float32)
    y, a = orc.linear_ref(x.view(np.uint16), wd)
    xd = x.astype(np.float64)
    want = xd @ wd.astype(np.float64).T
    want_a = np.abs(xd) @ np.abs(wd.astype(np.float64)).T
    assert np.allclose(y, want, rtol=0, atol=1e-12 * want_a.max())
    assert np.allclose(a, want_a, rtol=1e-13, atol=0)
    # one-hot x picks one column of w' exactly
    k = 333
    onehot = np.zeros((1, n_in), dtype=np.float16)
    onehot[0, k] = 1.0
    y1, _ = orc.linear_ref(onehot.view(np.uint16), wd)
    assert np.array_equal(y1[0], wd[:, k].astype(np.float64))
    # a non-symmetric x and w catch a transposed operand
    x2 = np.zeros((2, n_in), dtype=np.float16)
    x2[1, 7] = 2.0
    y2, _ = orc.linear_ref(x2.view(np.uint16), wd)
    assert np.all(y2[0] == 0) and np.array_equal(y2[1], 2.0 * wd[:, 7].astype(np.float64))
    y0, a0 = orc.linear_ref(x.view(np.uint16), np.zeros_like(wd))
    assert np.all(y0 == 0) and np.all(a0 == 0)


# ---------------------------------------------------------------------------
# INT8 codes (W8A16) and per-channel groups ([Guide] §2.1 b-bit ranges,
# §2.2 per-channel for INT8 weights, §2.3 W8A16).
# ---------------------------------------------------------------------------
def _codes_b(packed, bits):
    per = 32 // bits
    shifts = (bits * np.arange(per, dtype=np.uint32))
    return ((packed[..., None] >> shifts) & ((1 << bits) - 1)).reshape(packed.shape[0], -1)


def pin_brute_force_int8_per_channel(orc, quick=False):
    cases = _small_cases()[:1] if quick else _small_cases()
    for ci, w in enumerate(cases):
        n_in = w.shape[1]
        for bits, g in ((8, 32), (8, n_in), (4, n_in)):
            for sym in (False, True):
                packed, scales, zeros, s32 = orc.quantize_pack(w, g, sym, bits=bits)
                assert packed.shape == (w.shape[0], n_in * bits // 32)
                assert scales.shape == (w.shape[0], n_in // g)
                try:
                    check_matrix(w, packed, scales, zeros, s32, g, sym, bits=bits)
                except AssertionError as e:
                    raise AssertionError(f"case {ci} bits={bits} g={g} sym={sym}: {e}") from None


def pin_ties_to_even_int8(orc, quick=False):
    # asymmetric: range [-127, 128] gives s = 255/255 = 1 exactly and z = 127
    vals = [-127.0, 128.0, 0.5, 1.5, 2.5, -0.5, -1.5, 3.5, -2.5, 100.5, -99.5] + [0.0] * 21
    w = np.array([vals], dtype=np.float32)
    for g in (32, 32):                               # one group == the whole row (per-channel)
        packed, scales, zeros, s32 = orc.quantize_pack(w, g, False, bits=8)
        assert float(s32[0, 0]) == 1.0 and float(_f16_bits_to_f32(zeros)[0, 0]) == 127.0
        codes = _codes_b(packed, 8)[0].tolist()
        want = [round(v) + 127 for v in vals]        # Python's round: half to even
        assert codes == want, f"int8 tie codes {codes[:11]} != {want[:11]}"
    # symmetric: max|w| = 127 gives s = 1; codes stored as q + 128
    vals_s = [127.0, -126.5, 0.5, 1.5, 2.5, -0.5, -3.5, 5.5, -127.0, 126.5] + [0.0] * 22
    w = np.array([vals_s], dtype=np.float32)
    packed, scales, zeros, s32 = orc.quantize_pack(w, 32, True, bits=8)
    assert float(s32[0, 0]) == 1.0 and float(_f16_bits_to_f32(zeros)[0, 0]) == 128.0
    codes = _codes_b(packed, 8)[0].tolist()
    assert codes == [round(v) + 128 for v in vals_s], f"int8 symmetric tie codes {codes[:10]}"


def pin_grid_exact_int8(orc, quick=False):
    rng = np.random.default_rng(42)
    rows, n_in = 12, 512
    w = np.empty((rows, n_in), dtype=np.float32)
    expect = []
    for r in range(rows):
        s = np.float32(np.float16(rng.uniform(1e-4, 0.02)))          # fp16-exact scale
        z = int(rng.integers(0, 256))
        u = rng.integers(0, 256, size=n_in)
        u[rng.integers(0, n_in)] = 0
        u[rng.integers(0, n_in)] = 255
        w[r] = s * (u - z).astype(np.float32)                        # exact in binary32
        expect.append((s, z, u))
    packed, scales, zeros, s32 = orc.quantize_pack(w, n_in, False, bits=8)   # per-channel
    codes = _codes_b(packed, 8)
    sh, zh = _f16_bits_to_f32(scales), _f16_bits_to_f32(zeros)
    for r, (s, z, u) in enumerate(expect):
        assert sh[r, 0] == s and zh[r, 0] == z, f"row {r}: (s, z) = ({sh[r, 0]}, {zh[r, 0]}) != ({s}, {z})"
        assert np.array_equal(codes[r], u), f"row {r}: int8 codes differ"
    wd = orc.dequant(packed, scales, zeros, n_in, bits=8)
    assert np.array_equal(wd.view(np.uint32), w.view(np.uint32)), "grid-exact int8 W not reproduced bitwise"


def pin_dequant_int8(orc, quick=False):
    rng = np.random.default_rng(72)
    n_out, n_in = 20, 384
    for g in (64, n_in):
        packed = rng.integers(0, 1 << 32, size=(n_out, n_in // 4), dtype=np.uint64).astype(np.uint32)
        s = rng.uniform(0, 0.01, size=(n_out, n_in // g)).astype(np.float16)
        s[0, 0] = 0.0
        s[1, 0] = np.float16(6e-8)                    # fp16 subnormal
        z = rng.integers(0, 256, size=(n_out, n_in // g)).astype(np.float16)
        got = orc.dequant(packed, s.view(np.uint16), z.view(np.uint16), g, bits=8)
        bytes_ = packed.view(np.uint8).reshape(n_out, n_in).astype(np.int64)   # little-endian bytes
        want = (s.astype(np.float32).repeat(g, axis=1)
                * (bytes_ - z.astype(np.int64).repeat(g, axis=1)).astype(np.float32))
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), f"int8 dequant g={g} differs bitwise"


def pin_reconstruction_bound_int8(orc, quick=False):
    rows = 16 if quick else 64
    w = synthetic.normal_weight(rows, 4096, seed=33, std=0.02, n_outlier_cols=8)
    for bits, g in ((8, 4096), (8, 128), (4, 4096)):
        for sym in (False, True):
            packed, scales, zeros, s32 = orc.quantize_pack(w, g, sym, bits=bits)
            wd = orc.dequant(packed, scales, zeros, g, bits=bits)
            s = s32.astype(np.float64).repeat(g, axis=1)
            sh = _f16_bits_to_f32(scales).astype(np.float64).repeat(g, axis=1)
            cmax = (1 << (bits - 1)) if sym else (1 << bits) - 1
            err = np.abs(w.astype(np.float64) - wd.astype(np.float64))
            bound = s * (0.5 + 2.0 ** -18) + cmax * np.abs(s - sh)
            bad = err > bound
            assert not bad.any(), (f"bits={bits} g={g} sym={sym}: |w-w'| exceeds s/2 at "
                                   f"{np.argwhere(bad)[:3].tolist()}")


# ---------------------------------------------------------------------------
# KV-cache codec (the interview guide's §6): V per token, K per channel.
# ---------------------------------------------------------------------------
def _kv_cases():
    """fp16 bit patterns [blocks, t, d] with outlier channels, heavy tails,
    a zero token and a constant channel."""
    rng = np.random.default_rng(71)
    a = rng.standard_normal((3, 16, 32)).astype(np.float32)
    a[:, :, 5] *= 40.0                              # K-style outlier channel
    a[1, 3, :] = 0.0                                # an all-zero token
    a[2, :, 7] = 0.375                              # a constant channel
    b = (rng.standard_t(3, size=(2, 8, 48)) * 0.3).astype(np.float32)
    return [a.astype(np.float16).view(np.uint16), b.astype(np.float16).view(np.uint16)]


def _check_rows(vals_f32, q, s, bits, where):
    half = 1 << (bits - 1)
    for r in range(vals_f32.shape[0]):
        check_group(vals_f32[r], float(s[r]), half, [int(c) + half for c in q[r]], True,
                    f"{where} row {r}", bits=bits)


def pin_kv_brute_force(orc, quick=False):
    cases = _kv_cases()
    if quick:                                       # the first case's first two blocks
        cases = [cases[0][:2]]
    for ci, x in enumerate(cases):
        xf = _f16_bits_to_f32(x)
        blocks, t, d = x.shape
        for bits in (8, 4):
            q, s = orc.kv_quant_tokens(x, bits)
            assert q.shape == x.shape and s.shape == (blocks, t)
            _check_rows(xf.reshape(-1, d), q.reshape(-1, d), s.reshape(-1), bits, f"tokens case {ci} b{bits}")
            qc, sc = orc.kv_quant_channels(x, bits)
            assert qc.shape == x.shape and sc.shape == (blocks, d)
            for b in range(blocks):
                _check_rows(xf[b].T, qc[b].T, sc[b], bits, f"channels case {ci} block {b} b{bits}")


def pin_kv_worked_example(orc, quick=False):
    """A token whose largest channel is 100: the guide's §3 numbers (scale
    about 0.787, 0.5 -> 1 -> 0.787) come out of the per-token codec."""
    g = _golden("worked_example.json")
    rng = np.random.default_rng(72)
    row = rng.uniform(-3, 3, size=128).astype(np.float32)
    row[9] = g["max_abs"]
    row[40] = g["x"]
    x = row.astype(np.float16).view(np.uint16)[None, :]
    q, s = orc.kv_quant_tokens(x, g["bits"])
    tol = 0.5 * 10.0 ** (-g["scale_printed_digits"])
    assert abs(float(s[0]) - g["scale_printed"]) <= tol, f"scale {s[0]}"
    assert int(q[0, 40]) == g["q"] and int(q[0, 9]) == 127
    x_hat = float(np.float32(q[0, 40]) * s[0])               # the binary32 product
    assert abs(x_hat - g["x_hat_printed"]) <= tol, f"x_hat {x_hat}"
    back = orc.kv_dequant_tokens(q, s)                          # then fp16 for the cache consumer
    assert int(back[0, 40]) == int(np.float16(x_hat).view(np.uint16))


def pin_kv_transpose(orc, quick=False):
    """K per channel over a block equals V per token on the transposed block."""
    for x in _kv_cases():
        for bits in (8, 4):
            qc, sc = orc.kv_quant_channels(x, bits)
            for b in range(x.shape[0]):
                qt, st = orc.kv_quant_tokens(np.ascontiguousarray(x[b].T), bits)
                assert np.array_equal(qc[b], qt.T), f"codes of block {b} differ"
                assert np.array_equal(sc[b].view(np.uint32), st.view(np.uint32)), f"scales of block {b} differ"


def pin_kv_bound(orc, quick=False):
    """|x - x'| <= s/2 plus the fp16 rounding of x', for both sides."""
    rng = np.random.default_rng(73)
    x = (rng.standard_normal((4, 64, 128)) * np.array([1.0] * 120 + [30.0] * 8)).astype(np.float16)
    xb = x.view(np.uint16)
    xf = x.astype(np.float64)
    for bits in (8, 4):
        q, s = orc.kv_quant_tokens(xb, bits)
        back = _f16_bits_to_f32(orc.kv_dequant_tokens(q, s)).astype(np.float64)
        bound = s.astype(np.float64)[..., None] * (0.5 + 2.0 ** -20) + np.abs(back) * 2.0 ** -11
        assert (np.abs(xf - back) <= bound).all(), f"tokens b{bits}: bound violated"
        qc, sc = orc.kv_quant_channels(xb, bits)
        back = _f16_bits_to_f32(orc.kv_dequant_channels(qc, sc)).astype(np.float64)
        bound = sc.astype(np.float64)[:, None, :] * (0.5 + 2.0 ** -20) + np.abs(back) * 2.0 ** -11
        assert (np.abs(xf - back) <= bound).all(), f"channels b{bits}: bound violated"
        # dequantization is the fp32 product, rounded once more to fp16
        want = (q.astype(np.float32) * s[..., None]).astype(np.float16).view(np.uint16)
        assert np.array_equal(orc.kv_dequant_tokens(q, s), want)


def pin_kv_ties_and_zero(orc, quick=False):
    # max |v| = 127 gives scale 1 exactly at 8 bits; half-integers round to even
    vals = [127.0, -126.5, 0.5, 1.5, 2.5, -0.5, -3.5, 5.5, 100.5, -0.0] + [0.0] * 6
    x = np.array([vals], dtype=np.float16).view(np.uint16)
    q, s = orc.kv_quant_tokens(x, 8)
    assert float(s[0]) == 1.0
    assert q[0].tolist() == [round(v) for v in vals], q[0].tolist()
    # 4 bits: max |v| = 7 gives scale 1
    vals4 = [7.0, -6.5, 0.5, 1.5, 2.5, -2.5, 3.5, 0.0]
    x4 = np.array([vals4], dtype=np.float16).view(np.uint16)
    q4, s4 = orc.kv_quant_tokens(x4, 4)
    assert float(s4[0]) == 1.0 and q4[0].tolist() == [round(v) for v in vals4], q4[0].tolist()
    # an all-zero token: the scale floor, every code 0, zeros back
    z = np.zeros((1, 64), dtype=np.uint16)
    qz, sz = orc.kv_quant_tokens(z, 8)
    assert float(sz[0]) == float(np.float32(1e-8)) and not qz.any()
    assert not orc.kv_dequant_tokens(qz, sz).any()


def pin_kv_cache_sizes(orc, quick=False):
    g = _golden("kv_cache.json")
    for e in g["entries"]:
        gb = orc.kv_cache_bytes(g["layers"], g["kv_heads"], g["head_dim"], g["seq"], g["batch"],
                                e["bits"]) / 1e9
        assert abs(gb - e["gb_printed"]) < 1.0, f"{e['bits']}-bit KV cache {gb:.1f} GB vs {e['gb_printed']}"
    # and the codes the codec writes occupy exactly that many bytes per element
    x = _kv_cases()[0]
    q, _ = orc.kv_quant_tokens(x, 8)
    assert q.nbytes * 2 == x.nbytes


# ---------------------------------------------------------------------------
# W8A8 with SmoothQuant (the interview guide's §4.2).
# ---------------------------------------------------------------------------
def _sq_case(seed, m=24, n=40, k=96):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((m, k)).astype(np.float32)
    x[:, rng.choice(k, 3, replace=False)] *= 60.0           # activation outlier channels
    w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    return x.astype(np.float16), w


def pin_sq_balance_and_limits(orc, quick=False):
    """alpha = 0.5 balances the channel maxima of X diag(s)^-1 and diag(s) W;
    alpha = 1 moves everything to the weights (activation maxima 1), alpha = 0
    leaves it in the activations (weight maxima 1).  Channel maxima by numpy."""
    x, w = _sq_case(81)
    a = np.abs(x.astype(np.float32)).max(axis=0)
    wm = np.abs(w).max(axis=0)
    assert np.array_equal(orc.col_absmax_f16(x.view(np.uint16)), a)
    assert np.array_equal(orc.col_absmax_f32(w), wm)
    s = orc.smooth_factors(a, wm, 0.5).astype(np.float64)
    np.testing.assert_allclose(a / s, wm * s, rtol=4e-7)
    s1 = orc.smooth_factors(a, wm, 1.0).astype(np.float64)
    np.testing.assert_allclose(a / s1, 1.0, rtol=4e-7)
    s0 = orc.smooth_factors(a, wm, 0.0).astype(np.float64)
    np.testing.assert_allclose(wm * s0, 1.0, rtol=4e-7)
    s3 = orc.smooth_factors(a, wm, 0.75).astype(np.float64)
    np.testing.assert_allclose(s3, a ** 0.75 / wm ** 0.25, rtol=2e-6)


def pin_sq_clamps(orc, quick=False):
    a = np.array([4.0, 0.0, 9.0, 0.0], dtype=np.float32)
    wm = np.array([0.0, 0.25, 1e-7, 0.0], dtype=np.float32)
    s = orc.smooth_factors(a, wm, 0.5).astype(np.float64)
    # weight maxima floored at 1e-5 before the power; s floored at 1e-5
    np.testing.assert_allclose(s, [2.0 / np.sqrt(1e-5), 1e-5, 3.0 / np.sqrt(1e-5), 1e-5], rtol=2e-7)


def pin_w8a8_row_quantizers(orc, quick=False):
    """Both INT8 row quantizers pass the brute-force check; with smoothing they
    equal the unsmoothed quantizer on numpy's binary32 w * s and x / s."""
    x, w = _sq_case(82)
    rows = 6 if quick else None                     # quick: the brute force on the first rows
    qw, sw = orc.w8a8_quant_weight(w)
    _check_rows(w[:rows], qw[:rows], sw[:rows], 8, "weights")
    qx, sx = orc.w8a8_quant_act(x.view(np.uint16))
    _check_rows(x.astype(np.float32)[:rows], qx[:rows], sx[:rows], 8, "activations")
    s = orc.smooth_factors(orc.col_absmax_f16(x.view(np.uint16)), orc.col_absmax_f32(w), 0.5)
    qws, sws = orc.w8a8_quant_weight(w, s)
    q2, s2 = orc.w8a8_quant_weight(w * s[None, :])
    assert np.array_equal(qws, q2) and np.array_equal(sws.view(np.uint32), s2.view(np.uint32))
    qxs, sxs = orc.w8a8_quant_act(x.view(np.uint16), s)
    xs = x.astype(np.float32) / s[None, :]
    for r in range(xs.shape[0]):
        sc, z, q = orc.quantize_group(xs[r], bits=8, symmetric=True)
        assert z == 0 and np.float32(sc) == sxs[r] and np.array_equal(q, qxs[r].astype(np.int32)), f"row {r}"


def pin_w8a8_gemm(orc, quick=False):
    rng = np.random.default_rng(83)
    qx = rng.integers(-128, 128, size=(17, 300)).astype(np.int8)
    qw = rng.integers(-128, 128, size=(23, 300)).astype(np.int8)
    ones_x, ones_w = np.ones(17, np.float32), np.ones(23, np.float32)
    y, acc = orc.w8a8_gemm(qx, ones_x, qw, ones_w)
    assert np.array_equal(acc, qx.astype(np.int64) @ qw.astype(np.int64).T)
    # small integer sums are exact in fp16; power-of-two scales scale exactly
    qs = (rng.integers(-3, 4, size=(5, 64))).astype(np.int8)
    ws = (rng.integers(-3, 4, size=(6, 64))).astype(np.int8)
    y, acc = orc.w8a8_gemm(qs, np.full(5, 0.25, np.float32), ws, np.full(6, 8.0, np.float32))
    assert np.array_equal(y.view(np.float16).astype(np.float64), (qs.astype(np.int64) @ ws.astype(np.int64).T) * 2.0)


def pin_w8a8_error_bound(orc, quick=False):
    """The smoothed W8A8 product against the binary64 X W^T: per element,
    |y - xw| <= sum_k (|x^_k| sw / 2 + |w^_k| sx / 2 + sx sw / 4) + fp16 rounding."""
    for seed in (84, 85):
        x, w = _sq_case(seed, m=32, n=48, k=256)
        s = orc.smooth_factors(orc.col_absmax_f16(x.view(np.uint16)), orc.col_absmax_f32(w), 0.5)
        qw, sw = orc.w8a8_quant_weight(w, s)
        qx, sx = orc.w8a8_quant_act(x.view(np.uint16), s)
        y, _ = orc.w8a8_gemm(qx, sx, qw, sw)
        yf = y.view(np.float16).astype(np.float64)
        xd, wd, sd = x.astype(np.float64), w.astype(np.float64), s.astype(np.float64)
        ref = xd @ wd.T
        xh, wh = np.abs(xd / sd), np.abs(wd * sd)
        sxd, swd = sx.astype(np.float64)[:, None], sw.astype(np.float64)[None, :]
        bound = (xh @ np.ones((xh.shape[1], 1))) * swd / 2 + sxd * (wh.sum(axis=1))[None, :] / 2
        bound += sxd * swd * x.shape[1] / 4 + np.abs(yf) * 2.0 ** -10 + 1e-6 * (np.abs(xd) @ np.abs(wd).T)
        assert (np.abs(yf - ref) <= bound).all(), f"seed {seed}: {np.abs(yf - ref).max()} vs bound"
        # and smoothing helps: the same product without smoothing has a larger worst error here
        qw0, sw0 = orc.w8a8_quant_weight(w)
        qx0, sx0 = orc.w8a8_quant_act(x.view(np.uint16))
        y0, _ = orc.w8a8_gemm(qx0, sx0, qw0, sw0)
        err0 = np.abs(y0.view(np.float16).astype(np.float64) - ref).max()
        assert np.abs(yf - ref).max() < err0, "smoothing should reduce the error on outlier activations"


# ---------------------------------------------------------------------------
# GPTQ (the interview guide's §4.3) and AWQ (§4.4).
# ---------------------------------------------------------------------------
def _calib(t, n, seed, outliers=2):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((t, n)).astype(np.float32)
    x[:, rng.choice(n, outliers, replace=False)] *= 8.0
    return x.astype(np.float16)


def _out_err(x, w, wd):
    xf = x.astype(np.float64)
    return float(np.sum((xf @ (w.astype(np.float64) - wd.astype(np.float64)).T) ** 2))


def pin_gptq_hessian_and_factor(orc, quick=False):
    """H = 2 X^T X, the damping adds 0.01 mean(diag H) to the diagonal, and U
    is upper triangular with a positive diagonal and U^T U = H^-1, which by
    uniqueness of the Cholesky factor makes it the factor the method names."""
    x = _calib(300, 96, 91)
    h = orc.gptq_hessian(x.view(np.uint16))
    xf = x.astype(np.float64)
    np.testing.assert_allclose(h, 2.0 * xf.T @ xf, rtol=1e-13, atol=1e-9)
    hd = orc.gptq_damp(h, 0.01)
    want = h + np.eye(96) * 0.01 * np.mean(np.diag(h))
    np.testing.assert_allclose(hd, want, rtol=1e-14)
    u = orc.gptq_hinv_chol(hd)
    assert np.array_equal(u, np.triu(u)) and (np.diag(u) > 0).all()
    hinv = np.linalg.inv(hd)
    np.testing.assert_allclose(u.T @ u, hinv, rtol=1e-9, atol=1e-12 * np.abs(hinv).max())


def pin_gptq_diagonal_hessian_is_rounding(orc, quick=False):
    """With a diagonal H the factor is diagonal, no error reaches another
    column, and GPTQ is plain round-to-nearest with the same groups."""
    w = synthetic.normal_weight(8, 256, seed=92, n_outlier_cols=2)
    u = np.diag(np.random.default_rng(93).uniform(0.5, 2.0, 256)).astype(np.float32)
    for g in (32, 128):
        for sym in (False, True):
            p, sc, z, _ = orc.gptq_quantize(w, u, g, 4, sym)
            pr, scr, zr, _ = orc.quantize_pack(w, g, sym)
            assert np.array_equal(p, pr) and np.array_equal(sc, scr) and np.array_equal(z, zr), (g, sym)


def _obq(w, hinv, g, bits=4):
    """The guide's OBQ statement, independently of the Cholesky form: for
    each column q the rest moves by -(w_q - quant(w_q)) / Hinv_qq * Hinv_q,rest,
    then q is eliminated from Hinv.  Group parameters come from the current
    weights with the asymmetric binary32 map; the error uses the fp16-stored
    scale.  Returns the codes and the compensated weights (binary64)."""
    w = w.astype(np.float64).copy()
    hinv = hinv.copy()
    n_out, n = w.shape
    codes = np.zeros((n_out, n), dtype=np.int64)
    s = np.zeros(n_out, dtype=np.float32)
    zz = np.zeros(n_out, dtype=np.int64)
    qmax = (1 << bits) - 1
    for q in range(n):
        for r in range(n_out):
            if q % g == 0:
                grp = w[r, q:q + g].astype(np.float32)
                mn, mx = np.float32(grp.min()), np.float32(grp.max())
                sc = max(np.float32((mx - mn) / np.float32(qmax)), np.float32(1e-8))
                s[r] = sc
                zz[r] = int(min(max(np.rint(np.float32(-mn / sc)), 0), qmax))
            c = int(min(max(np.rint(np.float32(np.float32(w[r, q]) / s[r])) + zz[r], 0), qmax))
            codes[r, q] = c
            deq = float(np.float16(s[r])) * (c - zz[r])
            e = (w[r, q] - deq) / hinv[q, q]
            w[r, q + 1:] -= e * hinv[q, q + 1:]
        hinv = hinv - np.outer(hinv[:, q], hinv[q, :]) / hinv[q, q]
    return codes, w


def pin_gptq_matches_obq(orc, quick=False):
    """Codes and compensated weights of the Cholesky-form column loop equal
    those of the explicit OBQ elimination (binary32 against binary64)."""
    rng = np.random.default_rng(94)
    w = (rng.standard_normal((4, 32)) * 0.02).astype(np.float32)
    x = _calib(200, 32, 95)
    h = orc.gptq_damp(orc.gptq_hessian(x.view(np.uint16)), 0.01)
    u = orc.gptq_hinv_chol(h).astype(np.float32)
    packed, _, _, w_comp = orc.gptq_quantize(w, u, 16, 4, False)
    codes = np.array([[(int(packed[r, k // 8]) >> (4 * (k % 8))) & 15 for k in range(32)] for r in range(4)])
    want_codes, want_w = _obq(w, np.linalg.inv(h), 16)
    assert np.array_equal(codes, want_codes), "codes differ from the OBQ elimination"
    scale = np.abs(w).max()
    assert np.abs(w_comp - want_w).max() <= 2e-5 * scale, np.abs(w_comp - want_w).max() / scale


def pin_gptq_lowers_output_error(orc, quick=False):
    for seed in (96, 97):
        w = synthetic.normal_weight(32, 256, seed=seed, n_outlier_cols=2)
        x = _calib(400, 256, seed + 10)
        for g in (32, 128):
            p, sc, z = orc.gptq(w, x.view(np.uint16), g)
            pr, scr, zr, _ = orc.quantize_pack(w, g)
            e_g = _out_err(x, w, orc.dequant(p, sc, z, g))
            e_r = _out_err(x, w, orc.dequant(pr, scr, zr, g))
            assert e_g < e_r, f"seed {seed} g={g}: GPTQ {e_g:.4g} vs rounding {e_r:.4g}"


def pin_awq(orc, quick=False):
    w = synthetic.normal_weight(24, 256, seed=98, n_outlier_cols=0)
    x = _calib(128, 256, 99, outliers=6)
    mean = orc.awq_act_mean(x.view(np.uint16))
    np.testing.assert_allclose(mean, np.abs(x.astype(np.float64)).mean(axis=0), rtol=1e-15)
    s = orc.awq_scales(mean, 0.5)
    np.testing.assert_allclose(s, np.maximum(mean ** 0.5, 1e-5), rtol=1e-7)
    assert (orc.awq_scales(np.zeros(3), 0.5) == np.float32(1e-5)).all()
    # alpha = 0: s = 1 and AWQ is plain rounding
    p0, s0, z0, w_eff0 = orc.awq_apply(w, orc.awq_scales(mean, 0.0), 128)
    pr, sr, zr, _ = orc.quantize_pack(w, 128)
    assert np.array_equal(p0, pr) and np.array_equal(s0, sr) and np.array_equal(z0, zr)
    # the loss is the squared output error on the calibration tokens
    p, sc, z, w_eff = orc.awq_apply(w, s, 128)
    loss = orc.awq_loss(x.view(np.uint16), w, w_eff)
    np.testing.assert_allclose(loss, _out_err(x, w, w_eff), rtol=1e-10)
    # and w_eff is the dequantized W diag(s) divided back by s
    np.testing.assert_allclose(w_eff * s[None, :], orc.dequant(p, sc, z, 128), rtol=2e-7, atol=1e-12)
    best, losses, s_b, *_ = orc.awq(w, x.view(np.uint16), 128)
    assert losses[best] == min(losses) and best == int(np.argmin(losses))
    assert losses[best] < losses[0], "scaling the salient channels should beat plain rounding here"


ALL_PINS = [
    pin_worked_example, pin_brute_force, pin_ties_to_even, pin_zero_clip,
    pin_reconstruction_bound, pin_idempotence, pin_grid_exact, pin_constant_groups,
    pin_storage_accounting, pin_f16_converter, pin_dequant, pin_linear_ref,
    pin_brute_force_int8_per_channel, pin_ties_to_even_int8, pin_grid_exact_int8,
    pin_dequant_int8, pin_reconstruction_bound_int8,
    pin_kv_brute_force, pin_kv_worked_example, pin_kv_transpose, pin_kv_bound, pin_kv_ties_and_zero,
    pin_kv_cache_sizes,
    pin_sq_balance_and_limits, pin_sq_clamps, pin_w8a8_row_quantizers, pin_w8a8_gemm, pin_w8a8_error_bound,
    pin_gptq_hessian_and_factor, pin_gptq_diagonal_hessian_is_rounding, pin_gptq_matches_obq,
    pin_gptq_lowers_output_error, pin_awq,
]
