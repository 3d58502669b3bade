"""Bit-exact number-format helpers for the CPU oracle (test infrastructure).

This module is part of the oracle: plain, slow, obviously-correct numpy code
that the tests, the smoke check and the benchmark's CPU-baseline leg use to
check the HIP library. Nothing in the product path may import it.

Every helper is written from a format definition, never from a vendor
library, and rounds with the plain "grid" method: find the spacing of the
target format at the value's binade, divide (an exact power-of-two scaling),
round half to even with ``np.rint`` and multiply back.

Formats
-------
* bfloat16: the upper 16 bits of an IEEE-754 binary32 (1 sign, 8 exponent,
  7 fraction bits; bias 127; subnormals, inf and NaN as in binary32).
* OCP FP8 E4M3 ("e4m3fn"), from the OCP 8-bit floating point specification:
  1 sign, 4 exponent, 3 fraction bits, bias 7, subnormals down to 2^-9, no
  infinities, a single NaN pattern per sign (S.1111.111), largest finite
  magnitude 448. The pages fix 448 as the FP8 range in the continuous
  ``amax / 448`` scale they replace ("[FP8][MoE] Honor UE8M0 activation
  scales in Triton MoE", Motivation).
* UE8M0: an unsigned 8-bit power-of-two scale, code = exponent + 127. The
  pages require the FP32 activation scales to be powers of two
  ("[FP8][MoE] Honor UE8M0 activation scales in Triton MoE", Motivation and
  the "More context" comment).
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0          # largest finite OCP E4M3 magnitude: 1.75 * 2^8
BF16_QNAN = 0x7FC0        # the canonical quiet NaN bit pattern used for padding
UE8M0_MIN_EXP = -127
UE8M0_MAX_EXP = 127


def _round_to_grid(x: np.ndarray, mant_bits: int, min_exp: int) -> np.ndarray:
    """Round float64 ``x`` to nearest-even on a binary grid with ``mant_bits``
    stored fraction bits whose smallest normal exponent is ``min_exp``
    (below it the spacing stays 2^(min_exp - mant_bits): subnormals).
    Infinities and NaNs pass through; no overflow handling here."""
    x = np.asarray(x, dtype=np.float64)
    out = x.copy()
    fin = np.isfinite(x) & (x != 0)
    # frexp: x = m * 2^E with 0.5 <= |m| < 1, so floor(log2|x|) = E - 1 exactly.
    _, E = np.frexp(x[fin])
    e = np.maximum(E - 1, min_exp)
    ulp = np.ldexp(1.0, e - mant_bits)
    out[fin] = np.rint(x[fin] / ulp) * ulp   # x/ulp and *ulp are exact scalings
    return out


def bf16_round(x) -> np.ndarray:
    """Round float32/float64 values once, nearest-even, to the bfloat16 grid.

    Returns float64 values that are exactly representable in bfloat16.
    Magnitudes that round beyond the largest finite bfloat16 become +-inf;
    NaN stays NaN."""
    r = _round_to_grid(x, 7, -126)
    big = np.isfinite(r) & (np.abs(r) >= 2.0 ** 128)
    r[big] = np.copysign(np.inf, r[big])
    return r


def bf16_bits(x) -> np.ndarray:
    """bfloat16 bit patterns (uint16) of ``x`` after one nearest-even rounding.

    NaN inputs map to the quiet NaN 0x7FC0 carrying the input's sign."""
    x = np.asarray(x, dtype=np.float64)
    r = bf16_round(x)
    nan = np.isnan(r)
    r32 = r.astype(np.float32)            # exact: r is on the bfloat16 grid
    bits = (r32.view(np.uint32) >> 16).astype(np.uint16)
    if nan.any():
        sign = (np.signbit(x[nan]).astype(np.uint16) << 15)
        bits[nan] = sign | np.uint16(BF16_QNAN)
    return bits


def bf16_to_f32(bits) -> np.ndarray:
    """Widen bfloat16 bit patterns to float32 (exact)."""
    b = np.asarray(bits).astype(np.uint16).astype(np.uint32) << 16
    return b.view(np.float32)


def bf16_to_f64(bits) -> np.ndarray:
    """Widen bfloat16 bit patterns to float64 (exact; NaN stays NaN)."""
    with np.errstate(invalid="ignore"):
        return bf16_to_f32(bits).astype(np.float64)


def e4m3_decode(codes) -> np.ndarray:
    """Value (float64) of OCP E4M3 codes: s.eeee.mmm, bias 7.
    Field e == 0 is subnormal m * 2^-9; S.1111.111 is NaN."""
    c = np.asarray(codes).astype(np.uint8).astype(np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.ldexp(1.0, e - 7))
    val = s * mag
    val = np.where((e == 15) & (m == 7), np.nan, val)
    return val


def e4m3_encode(x) -> np.ndarray:
    """OCP E4M3 code (uint8) of float64 ``x``: one nearest-even rounding,
    subnormals kept, the sign of zero kept (-0 -> 0x80).

    Values whose rounded magnitude exceeds 448, and NaN, give the NaN code
    (0x7F / 0xFF); the finalize quantizer never produces them because it
    scales every block into [-448, 448] first."""
    x = np.asarray(x, dtype=np.float64)
    r = _round_to_grid(x, 3, -6)
    sign = np.signbit(x).astype(np.int64) << 7
    a = np.abs(r)
    code = np.zeros(x.shape, dtype=np.int64)
    nz = np.isfinite(a) & (a != 0) & (a <= E4M3_MAX)
    _, E = np.frexp(a[nz])
    e_unb = E - 1                                    # floor(log2 a)
    sub = e_unb < -6
    field = np.where(sub, 0, e_unb + 7)
    frac = np.where(sub, a[nz] * 2.0 ** 9,          # subnormal: m = a / 2^-9
                    (a[nz] / np.ldexp(1.0, e_unb) - 1.0) * 8.0)
    code[nz] = (field << 3) | np.rint(frac).astype(np.int64)
    bad = ~np.isfinite(a) | (a > E4M3_MAX)
    code[bad] = 0x7F
    return (code | sign).astype(np.uint8)


def ue8m0_exponent(amax) -> np.ndarray:
    """Power-of-two block-scale exponent for a block whose largest magnitude
    is ``amax`` (float64 array): the least integer e with amax <= 448 * 2^e,
    so the block scaled by 2^-e fits the E4M3 range and the scale is the
    power of two 2^ceil(log2(amax / 448)).

    Conventions: amax == 0 gives -127; the result is clamped to
    [-127, 127]; a non-finite amax gives 127."""
    a = np.asarray(amax, dtype=np.float64)
    e = np.full(a.shape, UE8M0_MIN_EXP, dtype=np.int64)
    pos = np.isfinite(a) & (a > 0)
    ap = a[pos]
    guess = np.ceil(np.log2(ap / E4M3_MAX)).astype(np.int64)
    # make the guess exact with comparisons that are exact in float64
    # (448 * 2^e and amax are both exactly representable)
    guess = np.where(ap > E4M3_MAX * np.ldexp(1.0, guess), guess + 1, guess)
    guess = np.where(ap <= E4M3_MAX * np.ldexp(1.0, guess - 1), guess - 1, guess)
    e[pos] = guess
    e[~np.isfinite(a)] = UE8M0_MAX_EXP
    return np.clip(e, UE8M0_MIN_EXP, UE8M0_MAX_EXP)


def ue8m0_code(exponent) -> np.ndarray:
    """UE8M0 byte for a power-of-two exponent: exponent + 127."""
    return (np.asarray(exponent, dtype=np.int64) + 127).astype(np.uint8)
