"""Pins for oracle.rmsnorm_bf16 (the q/k/v projection's input before quantization).

h = BF16(x / sqrt(mean(x^2) + eps) * gamma) is pinned against a 60-digit decimal
evaluation rounded to BF16 with exact rational arithmetic (which catches a sum in
place of the mean, eps outside the root, or an intermediate BF16 rounding), and
against closed forms.
"""

import decimal
from fractions import Fraction

import numpy as np

import oracle
import synth
from tests.exact import bf16_bits_of, bf16_to_fraction, round_to_bf16

EPS = np.float32(1e-5)


def rmsnorm_exact_bits(x_row, g_row, eps):
    ctx = decimal.Context(prec=60)
    xs = [bf16_to_fraction(int(b)) for b in x_row]
    gs = [bf16_to_fraction(int(b)) for b in g_row]
    ms = sum(x * x for x in xs) / len(xs) + Fraction(float(np.float32(eps)))
    msd = ctx.divide(decimal.Decimal(ms.numerator), decimal.Decimal(ms.denominator))
    r = Fraction(ctx.divide(decimal.Decimal(1), ctx.sqrt(msd)))
    out = []
    for xb, gb, x, g in zip(x_row, g_row, xs, gs):
        h = x * r * g
        bits = bf16_bits_of(float(round_to_bf16(h)))
        if h < 0 or (h == 0 and ((int(xb) ^ int(gb)) & 0x8000)):
            bits |= 0x8000
        out.append(bits)
    return np.array(out, dtype=np.uint16)


def bf16(a):
    a = np.asarray(a, dtype=np.float32)
    return synth.f32_to_bf16_bits(a).reshape(a.shape)


def test_rmsnorm_matches_exact_decimal():
    rng = np.random.default_rng(41)
    for K in (8, 32, 128, 256):
        x = bf16(rng.standard_normal((6, K)) * 10.0 ** rng.integers(-20, 20, (6, 1)))
        g = bf16(rng.standard_normal(K) * 0.7 + 1.0)
        got = oracle.rmsnorm_bf16(x, g, EPS)
        for m in range(x.shape[0]):
            want = rmsnorm_exact_bits(x[m], g, EPS)
            assert np.array_equal(got[m], want), (K, m, np.flatnonzero(got[m] != want)[:5])


def test_rmsnorm_closed_forms():
    K = 64
    g = bf16(np.linspace(-2, 2, K))
    # all-zero row: h = +-0 with the sign of x * gamma
    h = oracle.rmsnorm_bf16(np.zeros((1, K), np.uint16), g, EPS)
    assert np.all((h & 0x7FFF) == 0)
    assert np.array_equal(h[0] >> 15, (g >> 15).astype(np.uint16))
    # +-c everywhere with eps negligible against c^2: h = +-gamma exactly
    x = np.where(np.arange(K) % 2 == 0, bf16(4096.0), bf16(-4096.0)).astype(np.uint16)[None, :]
    h = oracle.rmsnorm_bf16(x, g, EPS)
    want = np.where(np.arange(K) % 2 == 0, g, g ^ np.uint16(0x8000))
    nz = (g & 0x7FFF) != 0
    assert np.array_equal(h[0][nz], want[nz])
    # scaling x by a power of two with eps far below mean(x^2) leaves h unchanged
    rng = np.random.default_rng(5)
    x = bf16(rng.standard_normal((4, K)) * 100)
    assert np.array_equal(oracle.rmsnorm_bf16(x, g, EPS), oracle.rmsnorm_bf16(bf16(
        oracle.bf16_bits_to_f32(x) * 4), g, EPS))


def test_rmsnorm_quant_is_quant_of_rmsnorm():
    rng = np.random.default_rng(8)
    x = bf16(rng.standard_normal((3, 512)))
    g = bf16(rng.standard_normal(512) * 0.1 + 1)
    q, s = oracle.rmsnorm_quant(x, g, EPS)
    q2, s2 = oracle.quant_act(oracle.rmsnorm_bf16(x, g, EPS))
    assert np.array_equal(q, q2) and np.array_equal(s, s2)
