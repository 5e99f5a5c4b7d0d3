"""Pins for oracle.silu_mul_bf16 / f64_to_bf16_bits (the down projection's input).

h = BF16(silu(g) * u) is pinned against a 60-digit decimal evaluation of
g / (1 + e^-g) * u rounded to BF16 with exact rational arithmetic, and against
closed-form special cases.
"""

import decimal
from fractions import Fraction

import numpy as np

import oracle
import synth
from tests.exact import bf16_bits_of, bf16_to_fraction, round_to_bf16


def silu_mul_exact_bits(g_bits, u_bits):
    ctx = decimal.Context(prec=60)
    g = bf16_to_fraction(g_bits)
    u = bf16_to_fraction(u_bits)
    gd = ctx.divide(decimal.Decimal(g.numerator), decimal.Decimal(g.denominator))
    e = ctx.exp(-gd)
    silu = ctx.divide(gd, ctx.add(decimal.Decimal(1), e))
    h = Fraction(silu) * u
    r = round_to_bf16(h)
    neg = h < 0 or (h == 0 and ((g_bits ^ u_bits) & 0x8000) and g != 0 and u != 0)
    bits = bf16_bits_of(float(r))
    if r == 0 and neg:
        bits |= 0x8000
    return bits


def test_f64_to_bf16_matches_exact_rounding():
    rng = np.random.default_rng(30)
    vals = np.concatenate([
        rng.standard_normal(3000) * 10.0 ** rng.integers(-40, 38, 3000),
        [1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, 2.0 ** -134, 3 * 2.0 ** -134, 2.0 ** -133 * 0.75, -0.0, 0.0],
    ])
    got = oracle.f64_to_bf16_bits(vals)
    for v, b in zip(vals, got):
        r = round_to_bf16(Fraction(float(v)))
        want = bf16_bits_of(float(r))
        if r == 0 and np.signbit(v):
            want |= 0x8000
        assert int(b) == want, v


def test_silu_mul_matches_high_precision_reference():
    rng = np.random.default_rng(31)
    M, I = 4, 256
    g = rng.standard_normal((M, I)).astype(np.float32) * np.float32(1.7)
    g[0, :8] = [0.0, -0.0, 80.0, -80.0, 1e-30, -1e-30, 3e4, -3e4]
    u = rng.standard_normal((M, I)).astype(np.float32) * np.float32(1.7)
    gu = np.concatenate([synth.f32_to_bf16_bits(g).reshape(M, I), synth.f32_to_bf16_bits(u).reshape(M, I)], axis=1)
    h = oracle.silu_mul_bf16(gu)
    assert h.shape == (M, I)
    for m in range(M):
        for i in range(I):
            want = silu_mul_exact_bits(int(gu[m, i]), int(gu[m, I + i]))
            got = int(h[m, i])
            if want & 0x7FFF == 0 and got & 0x7FFF == 0:
                continue            # the sign of an exact zero is not part of the contract
            assert got == want, (m, i)


def test_silu_special_values():
    one = 0x3F80
    gu = np.array([[0x0000, 0x4120, 0xC120, one, one, one]], dtype=np.uint16)   # g = 0, 10, -10; u = 1
    h = oracle.bf16_bits_to_f32(oracle.silu_mul_bf16(gu))[0]
    assert h[0] == 0
    assert abs(h[1] - 10.0) <= 10.0 * 2 ** -8          # silu(10) = 9.99955
    assert -0.00046 < h[2] < -0.00045                  # silu(-10) = -4.54e-4


def test_silu_mul_quant_is_quant_of_h():
    rng = np.random.default_rng(32)
    gu = synth.f32_to_bf16_bits(rng.standard_normal((2, 512)).astype(np.float32)).reshape(2, 512)
    q, s = oracle.silu_mul_quant(gu)
    q2, s2 = oracle.quant_act(oracle.silu_mul_bf16(gu))
    assert np.array_equal(q, q2) and np.array_equal(s, s2) and q.shape == (2, 256)


def test_silu_mul_near_rounding_midpoints():
    """Inputs whose product lies within 2^-12 of a BF16 rounding midpoint (relative to the
    BF16 quantum): an evaluation carried in float32, or any second rounding, errs on
    many of them; the decimal reference decides."""
    rng = np.random.default_rng(33)
    n = 1 << 21
    gb = synth.f32_to_bf16_bits(rng.standard_normal(n).astype(np.float32) * np.float32(2.0))
    ub = synth.f32_to_bf16_bits(rng.standard_normal(n).astype(np.float32) * np.float32(2.0))
    g = oracle.bf16_bits_to_f32(gb).astype(np.float64)
    u = oracle.bf16_bits_to_f32(ub).astype(np.float64)
    h = g / (1.0 + np.exp(-g)) * u                        # selection only, not the check
    _, e = np.frexp(h)
    frac = np.ldexp(np.abs(h), -(np.maximum(e, -125) - 8)) % 1.0
    near = np.nonzero(np.abs(frac - 0.5) < 2.0 ** -12)[0][:300]
    assert near.size >= 100
    gu = np.stack([gb[near], ub[near]], axis=1).astype(np.uint16)
    got = oracle.silu_mul_bf16(gu)[:, 0]
    for i in range(near.size):
        want = silu_mul_exact_bits(int(gu[i, 0]), int(gu[i, 1]))
        assert int(got[i]) == want, i
