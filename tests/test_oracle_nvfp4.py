"""Pins for oracle.nvfp4 (NVFP4 weight-only linear: E2M1 codes, E4M3 group-16
scales, float32 global scale, BF16 activations, float64 matmul).

Pinned against: the E2M1 value set of the OCP MX element format, a generic
minifloat decoder that is itself checked against torch's float8 decodes, an integer
bit loop for the nibble packing, an exact rational triple loop on small non-square
shapes, and closed-form special cases (single-column spikes at group edges, unit
codes and scales, power-of-two global scales).
"""

from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synth
from tests.exact import bf16_to_fraction, minifloat_exact

# Positive E2M1 values of the OCP MX element format (1 sign, 2 exponent, 1 mantissa bit).
E2M1_POSITIVE = [0, Fraction(1, 2), 1, Fraction(3, 2), 2, 3, 4, 6]


@pytest.mark.parametrize("dtype,ebits,mbits,bias", [(torch.float8_e4m3fn, 4, 3, 7), (torch.float8_e5m2, 5, 2, 15)])
def test_generic_minifloat_decoder_matches_torch(dtype, ebits, mbits, bias):
    codes = torch.arange(256, dtype=torch.uint8)
    vals = codes.view(dtype).to(torch.float64).numpy()
    n = 0
    for c in range(256):
        if not np.isfinite(vals[c]):
            continue
        assert Fraction(float(vals[c])) == minifloat_exact(c, ebits, mbits, bias), (dtype, c)
        n += 1
    assert n >= 248                                  # e5m2 has 8 infinity and NaN codes


def test_e2m1_table_is_the_format_definition():
    t = oracle.e2m1_decode_table()
    assert t.shape == (16,)
    for c in range(16):
        assert Fraction(float(t[c])) == minifloat_exact(c, 2, 1, 1), c
        mag = E2M1_POSITIVE[c & 7]
        assert Fraction(float(t[c])) == (-mag if c & 8 else mag), c
    assert np.signbit(t[8]) and t[8] == 0.0          # code 0x8 is -0
    assert t[7] == 6.0 and t[15] == -6.0             # no infinity or NaN: 0x7 is the largest


def test_unpack_nibble_order():
    assert oracle.unpack_fp4(np.array([[0x21]], np.uint8)).tolist() == [[1, 2]]
    rng = np.random.default_rng(40)
    p = rng.integers(0, 256, size=(3, 10), dtype=np.uint8)
    codes = oracle.unpack_fp4(p)
    assert codes.shape == (3, 20)
    for n in range(3):
        for k in range(20):
            assert codes[n, k] == (int(p[n, k // 2]) >> (4 * (k % 2))) & 0xF


def random_nvfp4(N, K, seed):
    rng = np.random.default_rng(seed)
    packed = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    # block scales over normal and subnormal E4M3 codes, some zero, positive only
    bs = rng.integers(0, 0x7F, size=(N, K // 16), dtype=np.uint8)
    bs[rng.random(bs.shape) < 0.1] = 0
    return packed, bs


def e4m3_exact(code):
    return minifloat_exact(code, 4, 3, 7)


def test_matches_exact_rational_triple_loop():
    M, K, N = 3, 96, 5
    rng = np.random.default_rng(41)
    xb = synth.f32_to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32)).reshape(M, K)
    packed, bs = random_nvfp4(N, K, 42)
    g = np.float32(3.7e-4)
    ref = oracle.linear_w4a16_ref(xb, packed, bs, g)
    assert ref.shape == (M, N)
    gq = Fraction(float(g))
    for m in range(M):
        for n in range(N):
            acc = Fraction(0)
            mag = Fraction(0)
            for k in range(K):
                code = (int(packed[n, k // 2]) >> (4 * (k & 1))) & 0xF
                t = bf16_to_fraction(xb[m, k]) * minifloat_exact(code, 2, 1, 1) * e4m3_exact(bs[n, k // 16]) * gq
                acc += t
                mag += abs(t)
            assert abs(Fraction(float(ref[m, n])) - acc) <= mag * Fraction(1, 2 ** 44) + Fraction(1, 2 ** 1074), (m, n)


@pytest.mark.parametrize("k", [0, 1, 14, 15, 16, 17, 31, 32, 47, 63])
def test_single_column_spike_picks_its_code_and_group_scale(k):
    # x is zero except column k, so y[n] = x[k] * e2m1(code[n, k]) * e4m3(bs[n, k // 16]) * g.
    K, N = 64, 4
    packed, bs = random_nvfp4(N, K, 43)
    bs[:, :] = np.arange(N * (K // 16), dtype=np.uint8).reshape(N, K // 16) + 0x30   # distinct per group
    x = np.zeros((1, K), np.float32)
    x[0, k] = 1.5
    xb = synth.f32_to_bf16_bits(x).reshape(1, K)
    g = np.float32(0.25)
    y = oracle.linear_w4a16_ref(xb, packed, bs, g)[0]
    for n in range(N):
        code = (int(packed[n, k // 2]) >> (4 * (k & 1))) & 0xF
        want = Fraction(3, 2) * E2M1_POSITIVE[code & 7] * (-1 if code & 8 else 1) * e4m3_exact(bs[n, k // 16]) / 4
        assert Fraction(float(y[n])) == want, (k, n)


def test_unit_codes_give_row_sums():
    M, K, N = 4, 128, 3
    xb = synth.bf16_normal(M, K, 1.0, seed=44, tid=synth.TID_X)
    packed = np.full((N, K // 2), 0x22, np.uint8)       # every code 2 = 1.0
    bs = np.full((N, K // 16), 0x38, np.uint8)          # E4M3 1.0
    y = oracle.linear_w4a16_ref(xb, packed, bs, np.float32(1.0))
    for m in range(M):
        s = sum(bf16_to_fraction(v) for v in xb[m])
        for n in range(N):
            assert abs(Fraction(float(y[m, n])) - s) <= sum(abs(bf16_to_fraction(v)) for v in xb[m]) * Fraction(1, 2 ** 50)


def test_global_scale_and_signs():
    M, K, N = 2, 64, 6
    xb = synth.bf16_normal(M, K, 1.0, seed=45, tid=synth.TID_X)
    packed, bs = random_nvfp4(N, K, 46)
    y1 = oracle.linear_w4a16_ref(xb, packed, bs, np.float32(1.0))
    y8 = oracle.linear_w4a16_ref(xb, packed, bs, np.float32(0.125))
    np.testing.assert_array_equal(y8, y1 * 0.125)       # power-of-two scaling is exact
    neg = packed ^ np.uint8(0x88)                       # flip both sign bits of every byte
    np.testing.assert_array_equal(oracle.linear_w4a16_ref(xb, neg, bs, np.float32(1.0)), -y1)
    zero = np.zeros_like(bs)
    assert not oracle.linear_w4a16_ref(xb, packed, zero, np.float32(1.0)).any()


def test_shape_checks():
    with pytest.raises(ValueError):
        oracle.dequant_nvfp4(np.zeros((2, 8), np.uint8), np.zeros((2, 2), np.uint8), 1.0)   # K=16 needs [2, 1]
    with pytest.raises(ValueError):
        oracle.dequant_nvfp4(np.zeros((2, 8), np.uint8), np.full((2, 1), 0x7F, np.uint8), 1.0)   # NaN scale
