"""Pins for the oracle's number-format helpers (CPU only).

Each helper is checked against something other than itself: torch's CPU
casts (library routines), exact rational arithmetic with ``fractions``,
exhaustive enumeration of every bf16 / E4M3 bit pattern, and closed forms.
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import formats as F


# ----------------------------------------------------------------- helpers
def all_bf16_patterns():
    return np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)


def frac_round_bf16(q: Fraction) -> Fraction:
    """Exact nearest-even rounding of a rational to the bf16 grid (finite,
    in range), by integer arithmetic only."""
    if q == 0:
        return Fraction(0)
    s = -1 if q < 0 else 1
    a = abs(q)
    # e = floor(log2 a) exactly
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    e = max(e, -126)
    ulp = Fraction(2) ** (e - 7)
    m = a / ulp
    n = m.numerator // m.denominator
    rem = m - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return s * n * ulp


def frac_ceil_log2(q: Fraction) -> int:
    """Least integer e with q <= 2^e, for q > 0 (exact)."""
    e = q.numerator.bit_length() - q.denominator.bit_length()
    while Fraction(2) ** e < q:
        e += 1
    while Fraction(2) ** (e - 1) >= q:
        e -= 1
    return e


# -------------------------------------------------------------------- bf16
def test_bf16_matches_torch_cast_random_and_specials():
    rng = np.random.default_rng(1)
    u = rng.integers(0, 1 << 32, size=400_000, dtype=np.uint64).astype(np.uint32)
    x = u.view(np.float32)
    x = x[np.isfinite(x) & (np.abs(x) < np.float32(3.38e38))]
    ties = ((rng.integers(0, 1 << 16, 20000, dtype=np.uint32) << 16) | 0x8000).view(np.float32)
    ties = ties[np.isfinite(ties) & (np.abs(ties) < np.float32(3.38e38))]
    x = np.concatenate([x, ties, np.float32([0.0, -0.0, 1.0, -1.0, 1e-40, -1e-45])])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = F.bf16_bits(x)
    assert np.array_equal(got, ref)


def test_bf16_exact_rational_bruteforce_fp64_inputs():
    rng = np.random.default_rng(2)
    xs = np.concatenate([rng.standard_normal(3000) * np.exp2(rng.integers(-140, 120, 3000)),
                         # just above / below a bf16 tie, where fp64->fp32->bf16
                         # would double-round
                         1.0 + 2.0 ** -8 + np.array([2.0 ** -30, -2.0 ** -30, 0.0]),
                         np.array([3 * 2.0 ** -134, 2.0 ** -134, -(2.0 ** -126)])])
    got = F.bf16_round(xs)
    for x, g in zip(xs, got):
        assert Fraction(float(g)) == frac_round_bf16(Fraction(float(x))), x


def test_bf16_single_rounding_not_double():
    # 1 + 2^-8 + 2^-30: fp32 first would land on the tie 1 + 2^-8 and round
    # to even (1.0); one rounding goes up to 1 + 2^-7.
    x = np.array([1.0 + 2.0 ** -8 + 2.0 ** -30])
    assert F.bf16_round(x)[0] == 1.0 + 2.0 ** -7
    assert F.bf16_bits(x)[0] == 0x3F81


def test_bf16_widen_roundtrip_all_patterns():
    b = all_bf16_patterns()
    v = F.bf16_to_f32(b)
    fin = np.isfinite(v)
    assert np.array_equal(F.bf16_bits(v[fin]), b[fin])
    # NaN maps to the quiet NaN with the sign kept
    nanb = F.bf16_bits(np.array([np.nan, -np.nan]))
    assert (nanb[0] & 0x7FFF) == 0x7FC0


def test_bf16_overflow_to_inf():
    big = np.array([3.4e38, -3.4e38])
    r = F.bf16_round(big)
    assert np.isinf(r).all() and r[0] > 0 and r[1] < 0


# -------------------------------------------------------------------- e4m3
def test_e4m3_decode_closed_forms():
    d = F.e4m3_decode(np.array([0x00, 0x80, 0x01, 0x07, 0x08, 0x38, 0x7E, 0xFE, 0x7F, 0xFF]))
    assert d[0] == 0.0 and math.copysign(1, d[1]) == -1
    assert d[2] == 2.0 ** -9
    assert d[3] == 7 * 2.0 ** -9
    assert d[4] == 2.0 ** -6
    assert d[5] == 1.0
    assert d[6] == 448.0 == F.E4M3_MAX
    assert d[7] == -448.0
    assert np.isnan(d[8]) and np.isnan(d[9])


def test_e4m3_roundtrip_all_finite_codes():
    codes = np.arange(256, dtype=np.uint16).astype(np.uint8)
    vals = F.e4m3_decode(codes)
    fin = ~np.isnan(vals)
    assert fin.sum() == 254
    assert np.array_equal(F.e4m3_encode(vals[fin]), codes[fin])


def test_e4m3_exhaustive_bf16_vs_torch():
    b = all_bf16_patterns()
    v = F.bf16_to_f32(b)
    sel = np.isfinite(v) & (np.abs(v) <= 448.0)
    x = v[sel]
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = F.e4m3_encode(x.astype(np.float64))
    assert np.array_equal(got, ref)


def test_e4m3_nearest_even_bruteforce():
    table = F.e4m3_decode(np.arange(256).astype(np.uint8))
    finite_codes = [c for c in range(256) if not np.isnan(table[c])]
    rng = np.random.default_rng(3)
    xs = np.concatenate([rng.uniform(-448, 448, 4000),
                         rng.uniform(-2 ** -5, 2 ** -5, 4000),
                         # exact midpoints between neighbours
                         (table[0x10:0x7E] + table[0x11:0x7F]) / 2,
                         (table[0x00:0x08] + table[0x01:0x09]) / 2])
    got = F.e4m3_encode(xs)
    for x, g in zip(xs, got):
        best = min(abs(table[c] - x) for c in finite_codes)
        cands = [c for c in finite_codes if abs(table[c] - x) == best]
        # ties: even mantissa (code's low bit 0); the sign follows x
        cands = [c for c in cands if (c & 0x80) == (0x80 if np.signbit(x) else 0)] or cands
        if len(cands) > 1:
            cands = [c for c in cands if c % 2 == 0]
        assert table[g] == table[cands[0]], (x, g, cands)


def test_e4m3_keeps_sign_of_zero():
    c = F.e4m3_encode(np.array([0.0, -0.0, -1e-9, 1e-9]))
    assert list(c) == [0x00, 0x80, 0x80, 0x00]


# ------------------------------------------------------------------- UE8M0
def test_ue8m0_exhaustive_positive_bf16_exact():
    b = all_bf16_patterns()
    v = F.bf16_to_f64(b)
    sel = np.isfinite(v) & (v > 0)
    amax = v[sel]
    got = F.ue8m0_exponent(amax)
    for a, e in zip(amax, got):
        want = frac_ceil_log2(Fraction(float(a)) / 448)
        assert e == min(127, max(-127, want)), a


def test_ue8m0_integer_bit_rule_for_normals():
    # Independent formulation on the float32 bit fields: amax = 2^E * 1.f;
    # 448 = 2^8 * 1.75, so e = E - 8 + (1.f > 1.75).
    b = all_bf16_patterns()
    v = F.bf16_to_f32(b)
    u = v.view(np.uint32)
    expf = (u >> 23) & 0xFF
    sel = (u >> 31 == 0) & (expf > 0) & (expf < 255)
    mant = u[sel] & 0x7FFFFF
    rule = (expf[sel].astype(np.int64) - 127) - 8 + (mant > 0x600000)
    rule = np.clip(rule, -127, 127)
    assert np.array_equal(F.ue8m0_exponent(v[sel].astype(np.float64)), rule)


def test_ue8m0_closed_form_bracket_and_edges():
    rng = np.random.default_rng(4)
    a = np.exp2(rng.uniform(-100, 100, 20000))
    e = F.ue8m0_exponent(a)
    assert np.all(a <= 448 * np.exp2(e)) and np.all(a > 448 * np.exp2(e - 1))
    e = F.ue8m0_exponent(np.array([0.0, 448.0, 449.0, 224.0, 224.5, 1.0, 2.0 ** -133,
                                   3.3895313892515355e38, np.inf]))
    assert list(e) == [-127, 0, 1, -1, 0, -8, -127, 120, 127]
    assert list(F.ue8m0_code(np.array([-127, 0, 127]))) == [0, 127, 254]
