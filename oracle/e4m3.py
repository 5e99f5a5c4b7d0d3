"""OCP E4M3 ("e4m3fn") decode table and round-to-nearest-even encoder with saturation.

Test infrastructure: see the package docstring.

Format (OCP 8-bit Floating Point Specification, OFP8, E4M3): 1 sign bit, 4 exponent
bits with bias 7, 3 mantissa bits.  Exponent field 0 holds subnormals m * 2^-9;
otherwise the value is (1 + m/8) * 2^(e-7).  The all-ones pattern S.1111.111 is NaN;
there is no infinity, so the largest finite magnitude is 0x7E = 1.75 * 2^8 = 448.
The model card "Nanbeige4.3-33B FP8" (introduction) names E4M3 as the code format
of both weights and activations; the e4m3fn variant is the one its sibling draft
model card (branch list) names.

The encoder here is deliberately the plainest possible: find the nearest entry of
the table of the 127 non-negative finite magnitudes, break exact ties toward the
code whose mantissa LSB is 0, and saturate magnitudes above 448 to 448.  All
comparisons are done in float64, where every float32 input, every table entry and
every midpoint between neighbouring entries is exact.
"""

import numpy as np

MAX_CODE = 0x7E          # largest finite magnitude code
MAX_FINITE = 448.0       # its value


def decode_table():
    """float64[256]: the value of every E4M3 byte (NaN for 0x7F and 0xFF)."""
    vals = np.empty(256, dtype=np.float64)
    for code in range(256):
        sign = -1.0 if code & 0x80 else 1.0
        e = (code >> 3) & 0xF
        m = code & 0x7
        if e == 0xF and m == 0x7:
            vals[code] = np.nan
        elif e == 0:
            vals[code] = sign * m * 2.0 ** -9
        else:
            vals[code] = sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return vals


_TABLE = decode_table()
# Non-negative finite magnitudes, codes 0x00..0x7E, strictly increasing.
_MAGS = _TABLE[: MAX_CODE + 1].copy()
assert np.all(np.diff(_MAGS) > 0)


def decode(codes):
    """float64 values of an array of E4M3 bytes."""
    return _TABLE[np.asarray(codes, dtype=np.uint8)]


def encode_rne_sat(v):
    """E4M3 byte for each float32 value: nearest, ties to even, saturate at +-448.

    ``v`` must hold no NaN (the quantizer never produces one for finite input).
    The sign bit is taken from the IEEE sign of ``v``, so -0.0 and negative values
    that round to zero give 0x80.
    """
    v = np.asarray(v, dtype=np.float32)
    if np.isnan(v).any():
        raise ValueError("E4M3 encode: NaN input is outside the oracle's contract")
    a = np.abs(v.astype(np.float64))
    a = np.minimum(a, MAX_FINITE)                       # saturation
    hi = np.searchsorted(_MAGS, a, side="left")         # first magnitude >= a
    hi = np.minimum(hi, MAX_CODE)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _MAGS[lo]
    d_hi = _MAGS[hi] - a
    take_hi = (d_hi < d_lo) | ((d_hi == d_lo) & ((hi & 1) == 0))
    mag_code = np.where(take_hi, hi, lo).astype(np.uint8)
    # a == _MAGS[hi] exactly: d_hi == 0 < d_lo unless hi == 0 (then lo == hi).
    sign = np.signbit(v).astype(np.uint8) << 7
    return (mag_code | sign).astype(np.uint8)
