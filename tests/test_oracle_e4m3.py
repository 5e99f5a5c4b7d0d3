"""Pins for oracle.e4m3 (OCP OFP8 E4M3 decode / nearest-even encode with saturation).

Pinned against: closed-form code values of the format definition, torch's CPU
float8_e4m3fn conversion (a library routine), and an integer bit-manipulation
encoder written here independently of the oracle's table search.
"""

import numpy as np
import pytest
import torch

import oracle


def encode_bits_reference(v):
    """Independent E4M3 encoder by integer manipulation of the float32 bit pattern."""
    u = np.ascontiguousarray(v, dtype=np.float32).view(np.uint32).astype(np.uint64)
    sign = ((u >> 31) << 7).astype(np.uint64)
    a = u & 0x7FFFFFFF
    a = np.minimum(a, 0x43E00000)                       # 448.0: saturate
    E = a >> 23
    # Normal E4M3 (|v| >= 2^-6, biased fp32 exponent >= 121): keep 3 mantissa bits.
    base = (a >> 20) - (120 << 3)
    rem = a & 0xFFFFF
    up = (rem > 0x80000) | ((rem == 0x80000) & ((base & 1) == 1))
    code_n = base + up
    # Subnormal E4M3: the value in units of 2^-9, rounded to an integer, ties to even.
    mant = np.where(E > 0, (a & 0x7FFFFF) | 0x800000, a & 0x7FFFFF)
    sh = 141 - np.maximum(E, 1)                          # value * 2^9 = mant * 2^-sh
    sh = np.minimum(sh, 63)
    q = mant >> sh
    r = mant & ((np.uint64(1) << sh) - 1)
    half = np.uint64(1) << (sh - 1)
    code_s = q + ((r > half) | ((r == half) & ((q & 1) == 1)))
    code = np.where(E >= 121, code_n, code_s)
    return (code | sign).astype(np.uint8)


def torch_cast(v):
    return torch.from_numpy(np.ascontiguousarray(v, dtype=np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_closed_form_codes():
    t = oracle.decode_table()
    assert t[0x38] == 1.0
    assert t[0x7E] == 448.0
    assert t[0x08] == 2.0 ** -6          # smallest normal
    assert t[0x01] == 2.0 ** -9          # smallest subnormal
    assert t[0x07] == 7 * 2.0 ** -9      # largest subnormal
    assert t[0x00] == 0.0 and not np.signbit(t[0x00])
    assert t[0x80] == 0.0 and np.signbit(t[0x80])
    assert np.isnan(t[0x7F]) and np.isnan(t[0xFF])
    assert np.isfinite(t).sum() == 254
    assert t[0x40] == 2.0 and t[0x3F] == 1.875


def test_decode_matches_torch_library():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    lib = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    t = oracle.decode_table()
    nan = np.isnan(lib)
    assert np.array_equal(nan, np.isnan(t))
    assert np.array_equal(lib[~nan], t[~nan])
    assert np.array_equal(np.signbit(lib[~nan]), np.signbit(t[~nan]))


def test_every_finite_code_round_trips():
    t = oracle.decode_table()
    codes = np.array([c for c in range(256) if np.isfinite(t[c])], dtype=np.uint8)
    vals = t[codes].astype(np.float32)
    assert np.array_equal(oracle.encode_rne_sat(vals), codes)


def test_midpoints_round_to_even_and_neighbours_to_nearer():
    t = oracle.decode_table()
    mags = t[:0x7F]
    for c in range(0x7E):
        mid = np.float32((mags[c] + mags[c + 1]) / 2)      # exact: 5 significant bits
        assert float(mid) == (mags[c] + mags[c + 1]) / 2
        even = c if c % 2 == 0 else c + 1
        below = np.nextafter(mid, np.float32(0))
        above = np.nextafter(mid, np.float32(np.inf))
        got = oracle.encode_rne_sat(np.array([mid, below, above, -mid], dtype=np.float32))
        assert list(got) == [even, c, c + 1, even | 0x80], c


def test_saturation_and_signed_zero():
    v = np.array([448.0, 449.0, 463.9, 464.0, 1e4, 3e38, -1e9, 0.0, -0.0, -2.0 ** -11, 2.0 ** -11],
                 dtype=np.float32)
    got = oracle.encode_rne_sat(v)
    assert list(got) == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0x00, 0x80, 0x80, 0x00]
    with pytest.raises(ValueError):
        oracle.encode_rne_sat(np.array([np.nan], dtype=np.float32))


def test_exhaustive_nonnegative_float32_up_to_464():
    """Every float32 bit pattern in [2^-11, 464]: oracle == bit encoder == torch cast.

    Below 2^-11 every value is under a quarter of the smallest subnormal code and
    encodes to 0x00; that range is checked on a stride sample plus its top pattern.
    Torch maps values above 464 to NaN (no saturation), so the library comparison
    stops there; saturation above is checked separately.
    """
    first = int(np.array([2.0 ** -11], dtype=np.float32).view(np.uint32)[0])
    last = int(np.array([464.0], dtype=np.float32).view(np.uint32)[0])
    step = 1 << 22
    for lo in range(first, last + 1, step):
        bits = np.arange(lo, min(lo + step, last + 1), dtype=np.uint32)
        v = bits.view(np.float32)
        o = oracle.encode_rne_sat(v)
        assert np.array_equal(o, encode_bits_reference(v)), hex(lo)
        assert np.array_equal(o, torch_cast(v)), hex(lo)
    tiny = np.concatenate([np.arange(0, first, 1021, dtype=np.uint32), np.array([first - 1], np.uint32)])
    v = tiny.view(np.float32)
    o = oracle.encode_rne_sat(v)
    assert np.all(o == 0)
    assert np.array_equal(o, torch_cast(v))


def test_negative_values_sampled():
    rng = np.random.default_rng(1)
    bits = rng.integers(0x80000000, 0xC3E80000, size=2_000_000, dtype=np.uint32)
    v = bits.view(np.float32)
    o = oracle.encode_rne_sat(v)
    assert np.array_equal(o, encode_bits_reference(v))
    assert np.array_equal(o, torch_cast(v))


def test_bit_encoder_saturates_like_oracle_above_464():
    rng = np.random.default_rng(2)
    bits = rng.integers(0x43E80000, 0x7F800000, size=200_000, dtype=np.uint32)
    v = bits.view(np.float32)
    o = oracle.encode_rne_sat(np.concatenate([v, -v]))
    assert np.all(o[: v.size] == 0x7E) and np.all(o[v.size:] == 0xFE)
    assert np.array_equal(o, encode_bits_reference(np.concatenate([v, -v])))
