"""Pins for oracle.quant: activation and weight quantizers.

Each property is fixed by the scheme (model card "Nanbeige4.3-33B FP8",
introduction and "Recipe and calibration": E4M3, 128x128 weight blocks, dynamic
per-token group-128 activation scales, minmax scales) under the readings in the
oracle docstring, and is checked with arithmetic independent of the oracle:
exact rationals for the scale and the quotient, brute-force nearest-code search
over torch-decoded E4M3 values, and invariants that a dropped term, a wrong axis
or a wrong sign would break.
"""

from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth
from tests.exact import (bf16_to_fraction, e4m3_values_exact, nearest_e4m3_code, round_to_f32)

MAGS = e4m3_values_exact()


def bf16_from_f32(x):
    x = np.asarray(x, dtype=np.float32)
    return synth.f32_to_bf16_bits(x).reshape(x.shape)


def random_x(M, K, seed=0, sigma=1.0):
    rng = np.random.default_rng(seed)
    return bf16_from_f32(rng.standard_normal((M, K)).astype(np.float32) * np.float32(sigma))


def test_shapes_and_group_layout():
    x = random_x(3, 384)
    q, s = oracle.quant_act(x)
    assert q.shape == (3, 384) and q.dtype == np.uint8
    assert s.shape == (3, 3) and s.dtype == np.float32
    with pytest.raises(ValueError):
        oracle.quant_act(random_x(2, 200))


def test_scale_is_correctly_rounded_amax_over_448():
    """s == fl32(amax / 448) bit for bit, by exact rational rounding."""
    x = random_x(16, 1024, seed=3)
    # plus edge groups: tiny / subnormal / huge BF16 amax
    edge = np.zeros((4, 1024), dtype=np.uint16)
    edge[0, :128] = 0x0001        # smallest BF16 subnormal, 9.18e-41
    edge[0, 128:256] = 0x0080     # smallest BF16 normal
    edge[1, :128] = 0x7F7F        # largest finite BF16
    edge[1, 300] = 0xFF7F         # its negative, alone in group 2
    edge[2, :] = bf16_from_f32(np.linspace(-3, 3, 1024))
    edge[3, 5] = 0x8001           # a lone negative subnormal
    x = np.concatenate([x, edge])
    q, s = oracle.quant_act(x)
    xf = oracle.bf16_bits_to_f32(x).reshape(x.shape[0], -1, 128)
    for m in range(x.shape[0]):
        for g in range(x.shape[1] // 128):
            amax = max(abs(Fraction(float(v))) for v in xf[m, g])
            want = round_to_f32(amax / 448)
            assert float(s[m, g]) == want, (m, g)


def test_codes_are_nearest_e4m3_of_correctly_rounded_quotient():
    """For sampled elements: code == nearest E4M3 to fl32(x / s) (exact rationals)."""
    x = random_x(8, 1024, seed=4)
    x[0, :128] = 0x0001                          # group of equal subnormals
    x[1, 0] = bf16_from_f32(-1e-30)              # underflows to -0 inside its group
    q, s = oracle.quant_act(x)
    rng = np.random.default_rng(5)
    picks = [(0, k) for k in range(0, 128, 17)] + [(1, 0)]
    picks += [(int(rng.integers(8)), int(rng.integers(1024))) for _ in range(1500)]
    for m, k in picks:
        xv = bf16_to_fraction(x[m, k])
        sv = Fraction(float(s[m, k // 128]))
        assert sv != 0
        quot = round_to_f32(xv / sv)
        neg = (quot < 0) or (quot == 0 and xv < 0) or (x[m, k] & 0x8000 and quot == 0)
        want = nearest_e4m3_code(Fraction(quot), MAGS, neg)
        assert int(q[m, k]) == want, (m, k, quot)


def test_every_nonzero_group_has_a_448_code_and_no_larger():
    x = random_x(64, 2048, seed=6, sigma=0.37)
    q, s = oracle.quant_act(x)
    mag = (q & 0x7F).reshape(64, 16, 128)
    assert np.all(mag.max(axis=2) == 0x7E)
    assert not np.any(mag == 0x7F)


def test_zero_group_gives_zero_scale_and_zero_codes():
    x = random_x(3, 512, seed=7)
    x[0, 128:256] = 0                  # +0.0 group
    x[1, :] = 0x8000                   # a row of -0.0
    x[2, 384:] = 0
    x[2, 400] = 0x8000
    q, s = oracle.quant_act(x)
    assert s[0, 1] == 0 and not np.signbit(s[0, 1]) and np.all(q[0, 128:256] == 0)
    assert np.all(s[1] == 0) and np.all(q[1] == 0)
    assert s[2, 3] == 0 and np.all(q[2, 384:] == 0)
    assert np.all(s[0, [0, 2, 3]] > 0)


def test_negation_flips_sign_bits_only():
    x = random_x(4, 512, seed=8)
    q, s = oracle.quant_act(x)
    qn, sn = oracle.quant_act(x ^ np.uint16(0x8000))
    assert np.array_equal(s, sn)
    assert np.array_equal(qn, q ^ np.uint8(0x80))


def test_power_of_two_scaling_moves_only_the_scale():
    x = random_x(4, 512, seed=9)
    q, s = oracle.quant_act(x)
    x4 = bf16_from_f32(oracle.bf16_bits_to_f32(x) * np.float32(4.0))
    q4, s4 = oracle.quant_act(x4)
    assert np.array_equal(q4, q)
    assert np.array_equal(s4, s * np.float32(4.0))


def test_group_structure_spike():
    """A single non-zero element lands in exactly one group of one row."""
    for (m, k) in [(0, 0), (2, 127), (1, 128), (3, 511)]:
        x = np.zeros((4, 512), dtype=np.uint16)
        x[m, k] = bf16_from_f32(-3.0)
        q, s = oracle.quant_act(x)
        nz = np.argwhere(s != 0)
        assert nz.tolist() == [[m, k // 128]]
        assert s[m, k // 128] == np.float32(3.0) / np.float32(448.0)
        assert np.argwhere(q != 0).tolist() == [[m, k]] and q[m, k] == 0xFE


def test_dequantization_error_bound():
    """|dec(q) s - x| <= half an E4M3 step of x/s, times s (plus the fl32 quotient rounding)."""
    x = random_x(32, 1024, seed=10)
    q, s = oracle.quant_act(x)
    xf = oracle.bf16_bits_to_f32(x).astype(np.float64)
    srep = np.repeat(s.astype(np.float64), 128, axis=1)
    deq = oracle.decode(q) * srep
    v = np.abs(xf / srep)
    step = np.where(v >= 2.0 ** -6, 2.0 ** (np.floor(np.log2(np.maximum(v, 2.0 ** -6))) - 3), 2.0 ** -9)
    assert np.all(np.abs(deq - xf) <= (0.5 * step * (1 + 2.0 ** -20) + 2.0 ** -24 * v) * srep)


def test_nonfinite_input_raises():
    x = random_x(1, 128)
    x[0, 3] = 0x7F80   # +inf
    with pytest.raises(ValueError):
        oracle.quant_act(x)


# ---------------------------------------------------------------- weights

def test_weight_scale_grid_orientation_and_exactness():
    """Non-square grid (N/128=2, K/128=3) with one distinct magnitude per block."""
    N, K = 256, 384
    rng = np.random.default_rng(11)
    w = rng.standard_normal((N, K)).astype(np.float32) * np.float32(0.02)
    mult = np.array([[1, 16, 256], [4096, 2.0 ** 16, 2.0 ** 20]], dtype=np.float32)
    w *= np.kron(mult, np.ones((128, 128), np.float32))
    wb = bf16_from_f32(w)
    qw, ws = oracle.quant_weight(wb)
    assert ws.shape == (2, 3)
    wf = oracle.bf16_bits_to_f32(wb)
    for i in range(2):
        for j in range(3):
            blk = wf[128 * i:128 * i + 128, 128 * j:128 * j + 128]
            amax = max(abs(Fraction(float(v))) for v in blk.reshape(-1))
            assert float(ws[i, j]) == round_to_f32(amax / 448), (i, j)
            assert (qw[128 * i:128 * i + 128, 128 * j:128 * j + 128] & 0x7F).max() == 0x7E
    # scales grow with the block multipliers in the same orientation
    r = ws / ws[0, 0]
    assert np.all(np.abs(np.log2(r) - np.log2(mult)) < 1.0)


def test_weight_codes_exact_on_samples():
    N, K = 128, 256
    wb = random_x(N, K, seed=12, sigma=0.02)
    qw, ws = oracle.quant_weight(wb)
    rng = np.random.default_rng(13)
    for _ in range(800):
        n, k = int(rng.integers(N)), int(rng.integers(K))
        xv = bf16_to_fraction(wb[n, k])
        sv = Fraction(float(ws[n // 128, k // 128]))
        quot = round_to_f32(xv / sv)
        neg = bool(wb[n, k] & 0x8000)
        assert int(qw[n, k]) == nearest_e4m3_code(Fraction(quot), MAGS, neg)


def test_weight_block_is_not_a_row_group():
    """A spike in one row of a block sets that block's scale for every row of it."""
    wb = np.zeros((256, 256), dtype=np.uint16)
    wb[:, :] = bf16_from_f32(np.float32(0.01))
    wb[3, 200] = bf16_from_f32(np.float32(4.48))
    qw, ws = oracle.quant_weight(wb)
    assert ws[0, 1] == oracle.bf16_bits_to_f32(wb[3, 200]) / np.float32(448)
    assert ws[0, 0] == ws[1, 0] == ws[1, 1]
    assert qw[3, 200] == 0x7E
    assert np.all(qw[0:128, 128:256][qw[0:128, 128:256] != 0x7E] == qw[0, 128])
