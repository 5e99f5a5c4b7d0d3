"""Pins for oracle.linear (dequantize-and-matmul in float64, tolerance check).

The block-scaled GEMM's value has a plain definition (sum over k of the two
dequantized operands); it is checked here against an exact rational triple loop
on small non-square shapes (so a transposed scale grid, a wrong group index or a
dropped scale fails), and against closed-form special cases.
"""

from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth
from tests.exact import e4m3_values_exact

MAGS = e4m3_values_exact()


def dec_exact(code):
    c = int(code)
    v = MAGS[c & 0x7F] if (c & 0x7F) != 0x7F else None
    assert v is not None
    return -v if c & 0x80 else v


def random_operands(M, K, N, seed):
    rng = np.random.default_rng(seed)
    xb = synth.f32_to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32)).reshape(M, K)
    wf = rng.standard_normal((N, K)).astype(np.float32) * np.float32(0.02)
    # distinct magnitudes per block so that the scale grid orientation matters
    grid = (2.0 ** rng.integers(-3, 4, size=(N // 128, K // 128))).astype(np.float32)
    wf *= np.kron(grid, np.ones((128, 128), np.float32))
    wb = synth.f32_to_bf16_bits(wf).reshape(N, K)
    q, s = oracle.quant_act(xb)
    qw, ws = oracle.quant_weight(wb)
    return q, s, qw, ws


def test_matches_exact_rational_triple_loop():
    M, K, N = 3, 384, 256
    q, s, qw, ws = random_operands(M, K, N, seed=20)
    ref = oracle.linear_ref(q, s, qw, ws)
    assert ref.shape == (M, N)
    for m in range(M):
        for n in range(0, N, 7):
            acc = Fraction(0)
            mag = Fraction(0)
            for k in range(K):
                t = dec_exact(q[m, k]) * Fraction(float(s[m, k // 128])) * \
                    dec_exact(qw[n, k]) * Fraction(float(ws[n // 128, k // 128]))
                acc += t
                mag += abs(t)
            assert abs(Fraction(float(ref[m, n])) - acc) <= mag * Fraction(1, 2 ** 44), (m, n)


def test_identity_weights_return_dequantized_activations():
    M, K = 5, 128
    xb = synth.f32_to_bf16_bits(np.random.default_rng(21).standard_normal((M, K)).astype(np.float32)).reshape(M, K)
    q, s = oracle.quant_act(xb)
    qw = np.zeros((128, 128), np.uint8)
    np.fill_diagonal(qw, 0x38)               # E4M3 1.0
    ws = np.ones((1, 1), np.float32)
    ref = oracle.linear_ref(q, s, qw, ws)
    a = np.array([[float(dec_exact(q[m, k]) * Fraction(float(s[m, 0]))) for k in range(K)] for m in range(M)])
    assert np.array_equal(ref, a)


def test_zero_rows_give_exact_zero():
    q, s, qw, ws = random_operands(4, 256, 128, seed=22)
    q[2] = 0
    s[2] = 0
    ref = oracle.linear_ref(q, s, qw, ws)
    assert np.all(ref[2] == 0)
    assert np.all(np.abs(ref[[0, 1, 3]]).max(axis=1) > 0)


def test_negation_and_power_of_two_scaling():
    q, s, qw, ws = random_operands(3, 256, 256, seed=23)
    ref = oracle.linear_ref(q, s, qw, ws)
    assert np.array_equal(oracle.linear_ref(q ^ np.uint8(0x80), s, qw, ws), -ref)
    assert np.array_equal(oracle.linear_ref(q, s, qw, ws * np.float32(2)), 2 * ref)


def test_tolerance_check_boundaries():
    ref = np.array([[1.0, -2.0, 0.0, 4.0]])
    rms = np.sqrt(np.mean(ref ** 2))
    bound = 4e-3 * np.abs(ref) + 1e-3 * rms
    ok = oracle.check_tolerance(ref + 0.999 * bound, ref)
    assert ok["ok"] and ok["n_fail"] == 0 and ok["worst"] <= 1
    bad = oracle.check_tolerance(ref + 1.01 * bound * np.array([[0, 0, 1, 0]]), ref)
    assert not bad["ok"] and bad["n_fail"] == 1
    nan = oracle.check_tolerance(np.array([[1.0, -2.0, np.nan, 4.0]]), ref)
    assert not nan["ok"]
    # BF16 bit patterns are decoded before comparing
    bits = synth.f32_to_bf16_bits(ref.astype(np.float32)).reshape(ref.shape)
    assert oracle.check_tolerance(bits, ref)["ok"]
    with pytest.raises(ValueError):
        oracle.check_tolerance(ref[:, :2], ref)


def test_bf16_rounding_of_the_reference_passes_its_own_tolerance():
    """A correctly rounded BF16 output always meets the bound (2^-9 < 4e-3)."""
    q, s, qw, ws = random_operands(8, 512, 384, seed=24)
    ref = oracle.linear_ref(q, s, qw, ws)
    y = oracle.f64_to_bf16_bits(ref)
    assert oracle.check_tolerance(y, ref)["ok"]
