"""Dense pin of the quantizer's per-element arithmetic: code = E4M3_RNE(fl32(x / s)).

The scheme (model card "Nanbeige4.3-33B FP8", introduction and "Recipe and
calibration") quantizes each element by its group's minmax scale.  Under the
reading that the quotient is one IEEE float32 division, the code of an element is
a pure function of two BF16 numbers: the element x and its group's amax.  These
tests enumerate that function densely -- every BF16 x with |x| <= amax, both
signs, for about two thousand amax values covering every BF16 exponent -- and
compare the oracle's codes with an expected code computed independently of it:

  * s = fl32(amax / 448) and v = fl32(x / s) as a float64 division rounded to
    float32.  A float64 quotient of two float32 operands, rounded again to float32,
    is the correctly rounded float32 quotient because 53 >= 2 * 24 + 2 (Figueroa,
    "When is double rounding innocuous?", 1995); every disagreement with the oracle
    is re-decided with exact rational arithmetic anyway;
  * the code of v from torch's float8_e4m3fn cast, a library routine that rounds
    to nearest even and agrees with OCP E4M3 for |v| <= 464 (here |v| <= 449).

Quotients formed differently -- x * fl32(1 / s), or x * fl32(448 / amax) -- differ
from fl32(x / s) in one float32 ulp for a small fraction of pairs, which moves the
E4M3 code whenever the two straddle a rounding midpoint; a dense enumeration meets
thousands of such pairs.
"""

from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from tests.exact import bf16_to_fraction, e4m3_values_exact, nearest_e4m3_code, round_to_f32

MAGS = e4m3_values_exact()


def _amax_bits(per_exponent, seed):
    """BF16 bit patterns of positive amax values: for each of the 255 exponent fields
    of finite BF16 (0 = subnormal), mantissas 0x00 (0x01 for subnormals), 0x7F and
    ``per_exponent - 2`` seeded random ones."""
    rng = np.random.default_rng(seed)
    out = []
    for e in range(255):
        mants = {1 if e == 0 else 0, 0x7F}
        while len(mants) < per_exponent:
            mants.add(int(rng.integers(1 if e == 0 else 0, 128)))
        out += [(e << 7) | m for m in sorted(mants)]
    return np.array(out, dtype=np.uint16)


def _pairs(amax_bits):
    """(x bit patterns, amax bit pattern per element): every BF16 x with |x| <= amax,
    both signs (+0 and -0 included)."""
    xs, ams = [], []
    for a in amax_bits:
        mags = np.arange(0, int(a) + 1, dtype=np.uint16)
        x = np.concatenate([mags, mags | np.uint16(0x8000)])
        xs.append(x)
        ams.append(np.full(x.shape, a, dtype=np.uint16))
    return np.concatenate(xs), np.concatenate(ams)


def _expected_codes(x_bits, amax_bits):
    """Independent expected code of each (x, amax) pair (see the module docstring)."""
    x = (x_bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    a = (amax_bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    s = (a / 448.0).astype(np.float32)
    v = (x / s.astype(np.float64)).astype(np.float32)
    v = np.clip(v, -448.0, 448.0).astype(np.float32)
    codes = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return codes, s


def _exact_code(xb, ab):
    """The code of one pair by exact rational arithmetic (the tie-breaker)."""
    x = bf16_to_fraction(xb)
    s = round_to_f32(bf16_to_fraction(ab) / 448)
    quot = round_to_f32(x / Fraction(s))
    quot = max(min(quot, 448.0), -448.0)
    neg = quot < 0 or (quot == 0 and (int(xb) & 0x8000) != 0)
    return nearest_e4m3_code(Fraction(abs(quot)), MAGS, neg)


def _check(got, x_bits, amax_bits):
    want, _ = _expected_codes(x_bits, amax_bits)
    bad = np.nonzero(got != want)[0]
    # Every disagreement is decided exactly: the oracle must match the rational result.
    wrong = [(int(x_bits[i]), int(amax_bits[i]), int(got[i]), int(want[i])) for i in bad
             if int(got[i]) != _exact_code(x_bits[i], amax_bits[i])]
    assert not wrong, f"{len(wrong)} codes differ from E4M3(fl32(x/s)), first {wrong[:5]}"
    return len(bad)


def _act_layout(x_bits, amax_bits):
    """Pack pairs into [rows, 128] groups: slot 0 holds the group's amax, slots 1..127
    hold x values of that amax (the tail of an amax's run is padded with +0)."""
    xs, slots = [], []
    start = 0
    n = len(x_bits)
    while start < n:
        a = amax_bits[start]
        end = start
        while end < n and amax_bits[end] == a:
            end += 1
        run = x_bits[start:end]
        groups = (len(run) + 126) // 127
        block = np.zeros((groups, 128), dtype=np.uint16)
        block[:, 0] = a
        flat = block[:, 1:].reshape(-1)
        flat[: len(run)] = run
        block[:, 1:] = flat.reshape(groups, 127)
        pos = np.zeros((groups, 127), dtype=bool).reshape(-1)
        pos[: len(run)] = True
        xs.append(block)
        slots.append(np.concatenate([np.zeros((groups, 1), bool), pos.reshape(groups, 127)], axis=1))
        start = end
    return np.concatenate(xs), np.concatenate(slots)


@pytest.mark.slow
def test_activation_codes_every_bf16_x_for_2040_amax_values():
    amax = _amax_bits(8, seed=11)
    assert len(amax) >= 2000
    checked = 0
    for chunk in np.array_split(amax, 16):
        x_bits, a_bits = _pairs(chunk)
        groups, used = _act_layout(x_bits, a_bits)
        rows = groups.reshape(-1, 8 * 128) if len(groups) % 8 == 0 else None
        if rows is None:                                  # pad to whole rows of 8 groups
            pad = (-len(groups)) % 8
            groups = np.concatenate([groups, np.tile(groups[-1:], (pad, 1))])
            used = np.concatenate([used, np.zeros((pad, 128), bool)])
            rows = groups.reshape(-1, 8 * 128)
        q, s = oracle.quant_act(rows)
        got = q.reshape(-1, 128)[used]
        _, s_want = _expected_codes(groups[:, 0], groups[:, 0])
        assert np.array_equal(s.reshape(-1).view(np.uint32), s_want.view(np.uint32))
        _check(got, x_bits, a_bits)
        checked += len(x_bits)
    assert checked > 30_000_000


@pytest.mark.slow
def test_weight_codes_every_bf16_x_for_765_amax_values():
    """The same enumeration through the 128 x 128 block weight quantizer: each block's
    element (0, 0) is the amax, the rest are x values of that amax."""
    amax = _amax_bits(3, seed=12)
    x_bits, a_bits = _pairs(amax)
    per = 128 * 128 - 1
    blocks, used = [], []
    start = 0
    while start < len(x_bits):
        a = a_bits[start]
        end = start
        while end < len(x_bits) and a_bits[end] == a:
            end += 1
        run = x_bits[start:end]
        nb = (len(run) + per - 1) // per
        b = np.zeros((nb, 128 * 128), dtype=np.uint16)
        u = np.zeros((nb, 128 * 128), dtype=bool)
        b[:, 0] = a
        fb = b[:, 1:].reshape(-1)
        fb[: len(run)] = run
        b[:, 1:] = fb.reshape(nb, per)
        fu = np.zeros(nb * per, dtype=bool)
        fu[: len(run)] = True
        u[:, 1:] = fu.reshape(nb, per)
        blocks.append(b)
        used.append(u)
        start = end
    blocks = np.concatenate(blocks)
    used = np.concatenate(used)
    # Lay the blocks side by side along K: W [128, 128 * nblocks].
    nb = len(blocks)
    w = blocks.reshape(nb, 128, 128).transpose(1, 0, 2).reshape(128, nb * 128)
    qw, ws = oracle.quant_weight(w)
    got = qw.reshape(128, nb, 128).transpose(1, 0, 2).reshape(nb, -1)[used]
    _, s_want = _expected_codes(blocks[:, 0], blocks[:, 0])
    assert np.array_equal(ws.reshape(-1).view(np.uint32), s_want.view(np.uint32))
    _check(got, x_bits, a_bits)
    assert len(x_bits) > 20_000_000


def test_expected_path_matches_exact_arithmetic_on_a_sample():
    """The float64-then-float32 quotient and torch's cast agree with exact rational
    arithmetic on seeded pairs, near-ties included (x = amax, x = amax / 2^k)."""
    rng = np.random.default_rng(13)
    amax = _amax_bits(3, seed=14)
    a = rng.choice(amax, 3000)
    x = (rng.integers(0, 1 << 15, 3000).astype(np.uint32) * a.astype(np.uint32) >> 15).astype(np.uint16)
    x = np.concatenate([x, a, np.maximum(a.astype(np.int32) - 128 * 3, 0).astype(np.uint16)])
    a = np.concatenate([a, a, a])
    x = np.where(rng.integers(0, 2, len(x)) == 1, x | np.uint16(0x8000), x).astype(np.uint16)
    want, _ = _expected_codes(x, a)
    for i in range(len(x)):
        assert int(want[i]) == _exact_code(x[i], a[i]), (int(x[i]), int(a[i]))
