"""Exact-arithmetic helpers for pinning the oracle (test-only, independent of it).

Everything here works on Python integers and fractions.Fraction, so it shares no
floating-point code path with the numpy oracle or the HIP kernels.
"""

from fractions import Fraction
import math
import struct

import numpy as np


def f32_from_bits(b):
    return struct.unpack("<f", struct.pack("<I", int(b) & 0xFFFFFFFF))[0]


def bf16_to_fraction(bits):
    v = f32_from_bits(int(bits) << 16)
    return Fraction(v)


def _round_half_even(r):
    """Nearest integer to the Fraction r, ties to even."""
    fl = math.floor(r)
    rem = r - fl
    if rem > Fraction(1, 2):
        return fl + 1
    if rem < Fraction(1, 2):
        return fl
    return fl if fl % 2 == 0 else fl + 1


def _round_to_binary(r, mant_bits, min_exp):
    """Round a Fraction to the nearest value with ``mant_bits`` significant bits whose
    quantum is never below 2^(min_exp - mant_bits + 1) (IEEE-style gradual underflow),
    ties to even.  Returns a Fraction."""
    if r == 0:
        return Fraction(0)
    sign = -1 if r < 0 else 1
    a = abs(r)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    # now 2^e <= a < 2^(e+1)
    e = max(e, min_exp)
    quantum = Fraction(2) ** (e - mant_bits + 1)
    n = _round_half_even(a / quantum)
    return sign * n * quantum


def round_to_f32(r):
    """Correctly rounded float32 (ties to even, subnormals kept) of a Fraction, as float."""
    return float(_round_to_binary(Fraction(r), 24, -126))


def round_to_bf16(r):
    """Correctly rounded BF16 of a Fraction, as a Fraction."""
    return _round_to_binary(Fraction(r), 8, -126)


def bf16_bits_of(value):
    """BF16 bit pattern of a value that is exactly representable in BF16."""
    b = struct.unpack("<I", struct.pack("<f", float(value)))[0]
    assert b & 0xFFFF == 0, "value is not a BF16 value"
    return b >> 16


def e4m3_values_exact():
    """Exact Fractions of the 127 non-negative finite E4M3 magnitudes, obtained from
    torch's float8_e4m3fn decode (a library routine, independent of the oracle)."""
    import torch
    codes = torch.arange(0, 0x7F, dtype=torch.uint8)
    vals = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    return [Fraction(float(v)) for v in vals]


def nearest_e4m3_code(r, mags, negative):
    """Brute force: the E4M3 code nearest to |Fraction r| (ties: even code), saturating,
    with the sign bit set when ``negative`` (the IEEE sign of the quotient)."""
    sign = 0x80 if negative else 0
    a = min(abs(r), mags[-1])
    best, best_d = None, None
    for c, m in enumerate(mags):
        d = abs(a - m)
        if best_d is None or d < best_d or (d == best_d and c % 2 == 0):
            best, best_d = c, d
    return best | sign


def np_f32(x):
    return np.float32(x)


def minifloat_exact(code, ebits, mbits, bias):
    """Exact Fraction of a sign/exponent/mantissa code of a binary minifloat with
    gradual underflow (exponent field 0: m * 2^(1 - bias - mbits)), ignoring any
    infinity or NaN encodings.  A generic decoder written from the IEEE-style layout,
    checked against torch's float8 decodes before it is trusted for other formats."""
    c = int(code)
    sign = -1 if (c >> (ebits + mbits)) & 1 else 1
    e = (c >> mbits) & ((1 << ebits) - 1)
    m = c & ((1 << mbits) - 1)
    if e == 0:
        mag = Fraction(m) * Fraction(2) ** (1 - bias - mbits)
    else:
        mag = (1 + Fraction(m, 1 << mbits)) * Fraction(2) ** (e - bias)
    return sign * mag
