"""The pins catch plausible mistakes: each case plants one into the oracle (CPU only,
through monkeypatch) and expects at least one of the pin tests to fail."""

import numpy as np
import pytest

import oracle
import oracle.e4m3 as e4m3
import oracle.linear as linear
import oracle.nvfp4 as nvfp4
import oracle.quant as quant
import oracle.rmsnorm as rmsnorm
from tests import test_oracle_e4m3 as te
from tests import test_oracle_linear as tl
from tests import test_oracle_nvfp4 as tn
from tests import test_oracle_quant as tq
from tests import test_oracle_quotient as tqq
from tests import test_oracle_rmsnorm as tr
from tests import test_oracle_silu as ts


def _fails(fn):
    try:
        fn()
    except (AssertionError, ValueError):
        return True
    return False


def _encode_ties_away(v):
    v = np.asarray(v, dtype=np.float32)
    a = np.minimum(np.abs(v.astype(np.float64)), 448.0)
    mags = e4m3._MAGS
    hi = np.minimum(np.searchsorted(mags, a), 0x7E)
    lo = np.maximum(hi - 1, 0)
    take_hi = (mags[hi] - a) <= (a - mags[lo])
    return (np.where(take_hi, hi, lo).astype(np.uint8) | (np.signbit(v).astype(np.uint8) << 7))


def _encode_no_sign(v):
    return e4m3.encode_rne_sat(np.abs(np.asarray(v, dtype=np.float32)))


def _quant_groups_reciprocal(x, axes):
    amax = np.max(np.abs(x), axis=axes, keepdims=True)
    s = (amax * np.float32(1.0 / 448.0)).astype(np.float32)
    zero = s == 0
    with np.errstate(divide="ignore", invalid="ignore"):
        v = (x / np.where(zero, np.float32(1), s)).astype(np.float32)
    q = e4m3.encode_rne_sat(np.clip(v, -448, 448))
    q = np.where(np.broadcast_to(zero, q.shape), np.uint8(0), q).astype(np.uint8)
    return q, np.squeeze(s, axis=axes).astype(np.float32)


def _quant_groups_quotient(kind):
    """_quant_groups with the quotient formed as x * fl32(1 / s) ("reciprocal") or as
    x * fl32(448 / amax) ("inverse_scale"), guarded the way a kernel would guard it:
    groups with s < 2^-60 keep the division."""
    def f(x, axes):
        amax = np.max(np.abs(x), axis=axes, keepdims=True)
        s = (amax / np.float32(448)).astype(np.float32)
        zero = s == 0
        safe = np.where(zero, np.float32(1), s)
        with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
            if kind == "reciprocal":
                y = (np.float32(1) / safe).astype(np.float32)
            else:
                y = (np.float32(448) / np.where(zero, np.float32(1), amax)).astype(np.float32)
            fast = (x * y).astype(np.float32)
            exact = (x / safe).astype(np.float32)
        v = np.where(s >= np.float32(2.0 ** -60), fast, exact)
        q = e4m3.encode_rne_sat(np.clip(v, -448, 448))
        q = np.where(np.broadcast_to(zero, q.shape), np.uint8(0), q).astype(np.uint8)
        return q, np.squeeze(s, axis=axes).astype(np.float32)
    return f


def _quant_act_with(groups_fn):
    def f(x_bits):
        x_bits = np.asarray(x_bits, dtype=np.uint16)
        M, K = x_bits.shape
        q, s = groups_fn(quant.bf16_bits_to_f32(x_bits).reshape(M, K // 128, 128), (2,))
        return q.reshape(M, K), s.reshape(M, K // 128)
    return f


def _quant_weight_with(groups_fn):
    def f(w_bits):
        w_bits = np.asarray(w_bits, dtype=np.uint16)
        N, K = w_bits.shape
        q, s = groups_fn(quant.bf16_bits_to_f32(w_bits).reshape(N // 128, 128, K // 128, 128), (1, 3))
        return q.reshape(N, K), s.reshape(N // 128, K // 128)
    return f


def _quant_act_strided_groups(x_bits):
    M, K = x_bits.shape
    x = quant.bf16_bits_to_f32(x_bits).reshape(M, 128, K // 128)
    q, s = quant._quant_groups(x, axes=(1,))
    return q.reshape(M, K), s.reshape(M, K // 128)


def _dequant_weight_transposed(qw, ws):
    N, K = qw.shape
    w = e4m3.decode(qw).reshape(N // 128, 128, K // 128, 128)
    wsT = np.asarray(ws, np.float32).T.reshape(ws.shape)      # scrambled grid
    return (w * wsT.astype(np.float64)[:, None, :, None]).reshape(N, K)


def _dequant_act_no_scale(q, s):
    return e4m3.decode(q).astype(np.float64)


def _silu_wrong_sign(gu_bits):
    gu = quant.bf16_bits_to_f32(gu_bits).astype(np.float64)
    h = gu.shape[1] // 2
    g, u = gu[:, :h], gu[:, h:]
    with np.errstate(over="ignore"):
        return quant.f64_to_bf16_bits(g / (1.0 + np.exp(g)) * u)


def _silu_via_f32(gu_bits):
    gu = quant.bf16_bits_to_f32(gu_bits)
    h = gu.shape[1] // 2
    g, u = gu[:, :h], gu[:, h:]
    with np.errstate(over="ignore"):
        r = (g / (np.float32(1) + np.exp(-g)) * u).astype(np.float32)
    return quant.f64_to_bf16_bits(r.astype(np.float64))   # double rounding


def _rmsnorm_variant(sum_not_mean=False, eps_outside=False, round_normalized=False):
    def f(x_bits, gamma_bits, eps):
        x = quant.bf16_bits_to_f32(np.asarray(x_bits, np.uint16)).astype(np.float64)
        g = quant.bf16_bits_to_f32(np.asarray(gamma_bits, np.uint16)).astype(np.float64)
        ms = np.sum(x * x, axis=1, keepdims=True)
        if not sum_not_mean:
            ms = ms / x.shape[1]
        e = float(np.float32(eps))
        r = 1.0 / np.sqrt(ms) + e if eps_outside else 1.0 / np.sqrt(ms + e)
        n = x * r
        if round_normalized:                                  # BF16(BF16(x r) * gamma)
            n = quant.bf16_bits_to_f32(quant.f64_to_bf16_bits(n)).astype(np.float64)
        with np.errstate(divide="ignore", invalid="ignore"):
            return quant.f64_to_bf16_bits(n * g)
    return f


def _unpack_high_first(packed):
    p = np.asarray(packed, dtype=np.uint8)
    codes = np.empty((p.shape[0], 2 * p.shape[1]), dtype=np.uint8)
    codes[:, 0::2] = p >> 4
    codes[:, 1::2] = p & 0x0F
    return codes


def _e2m1_bias0():
    t = np.empty(16)
    for c in range(16):
        e, m = (c >> 1) & 3, c & 1
        v = m * 1.0 if e == 0 else (1 + m / 2) * 2.0 ** e
        t[c] = -v if c & 8 else v
    return t


def _e2m1_subnormal_as_normal():
    t = nvfp4.e2m1_decode_table().copy()
    t[1], t[9] = 0.75, -0.75                              # 2^(0-1) * (1 + 1/2)
    return t


def _dequant_nvfp4_variant(divide_g=False, strided=False, no_scale=False):
    def f(packed, bs, g):
        codes = nvfp4.unpack_fp4(packed)
        N, K = codes.shape
        sc = e4m3.decode(np.asarray(bs, np.uint8))
        if no_scale:
            sc = np.ones_like(sc)
        kk = np.arange(K)
        grp = (kk % (K // 16)) if strided else kk // 16
        w = nvfp4._E2M1[codes] * sc[:, grp]
        gv = float(np.float32(g))
        return w / gv if divide_g else w * gv
    return f


MUTATIONS = {
    "ties_away_from_zero": ([(e4m3, "encode_rne_sat", _encode_ties_away), (quant, "encode_rne_sat", _encode_ties_away),
                             (oracle, "encode_rne_sat", _encode_ties_away)],
                            [te.test_midpoints_round_to_even_and_neighbours_to_nearer]),
    "sign_dropped": ([(quant, "encode_rne_sat", _encode_no_sign)],
                     [tq.test_negation_flips_sign_bits_only]),
    "scale_by_reciprocal": ([(quant, "_quant_groups", _quant_groups_reciprocal)],
                            [tq.test_scale_is_correctly_rounded_amax_over_448]),
    "act_quotient_by_reciprocal": (
        [(quant, "quant_act", _quant_act_with(_quant_groups_quotient("reciprocal"))),
         (oracle, "quant_act", _quant_act_with(_quant_groups_quotient("reciprocal")))],
        [tqq.test_activation_codes_every_bf16_x_for_2040_amax_values]),
    "act_quotient_by_448_over_amax": (
        [(quant, "quant_act", _quant_act_with(_quant_groups_quotient("inverse_scale"))),
         (oracle, "quant_act", _quant_act_with(_quant_groups_quotient("inverse_scale")))],
        [tqq.test_activation_codes_every_bf16_x_for_2040_amax_values]),
    "weight_quotient_by_reciprocal": (
        [(quant, "quant_weight", _quant_weight_with(_quant_groups_quotient("reciprocal"))),
         (oracle, "quant_weight", _quant_weight_with(_quant_groups_quotient("reciprocal")))],
        [tqq.test_weight_codes_every_bf16_x_for_765_amax_values]),
    "weight_quotient_by_448_over_amax": (
        [(quant, "quant_weight", _quant_weight_with(_quant_groups_quotient("inverse_scale"))),
         (oracle, "quant_weight", _quant_weight_with(_quant_groups_quotient("inverse_scale")))],
        [tqq.test_weight_codes_every_bf16_x_for_765_amax_values]),
    "strided_groups": ([(quant, "quant_act", _quant_act_strided_groups), (oracle, "quant_act", _quant_act_strided_groups)],
                       [tq.test_group_structure_spike]),
    "weight_grid_transposed": ([(linear, "dequant_weight", _dequant_weight_transposed)],
                               [tl.test_matches_exact_rational_triple_loop]),
    "activation_scale_dropped": ([(linear, "dequant_act", _dequant_act_no_scale)],
                                 [tl.test_matches_exact_rational_triple_loop]),
    "silu_sign": ([(quant, "silu_mul_bf16", _silu_wrong_sign), (oracle, "silu_mul_bf16", _silu_wrong_sign)],
                  [ts.test_silu_special_values]),
    "silu_double_rounding": ([(quant, "silu_mul_bf16", _silu_via_f32), (oracle, "silu_mul_bf16", _silu_via_f32)],
                             [ts.test_silu_mul_matches_high_precision_reference, ts.test_silu_mul_near_rounding_midpoints]),
    "rmsnorm_sum_not_mean": ([(rmsnorm, "rmsnorm_bf16", _rmsnorm_variant(sum_not_mean=True)),
                              (oracle, "rmsnorm_bf16", _rmsnorm_variant(sum_not_mean=True))],
                             [tr.test_rmsnorm_matches_exact_decimal]),
    "rmsnorm_eps_outside_root": ([(rmsnorm, "rmsnorm_bf16", _rmsnorm_variant(eps_outside=True)),
                                  (oracle, "rmsnorm_bf16", _rmsnorm_variant(eps_outside=True))],
                                 [tr.test_rmsnorm_matches_exact_decimal, tr.test_rmsnorm_closed_forms]),
    "rmsnorm_double_rounding": ([(rmsnorm, "rmsnorm_bf16", _rmsnorm_variant(round_normalized=True)),
                                 (oracle, "rmsnorm_bf16", _rmsnorm_variant(round_normalized=True))],
                                [tr.test_rmsnorm_matches_exact_decimal]),
    "fp4_high_nibble_first": ([(nvfp4, "unpack_fp4", _unpack_high_first), (oracle, "unpack_fp4", _unpack_high_first)],
                              [tn.test_unpack_nibble_order]),
    "e2m1_bias_zero": ([(nvfp4, "_E2M1", _e2m1_bias0())],
                       [tn.test_matches_exact_rational_triple_loop]),
    "e2m1_subnormal_as_normal": ([(nvfp4, "_E2M1", _e2m1_subnormal_as_normal())],
                                 [tn.test_matches_exact_rational_triple_loop]),
    "nvfp4_global_scale_divides": ([(nvfp4, "dequant_nvfp4", _dequant_nvfp4_variant(divide_g=True))],
                                   [tn.test_matches_exact_rational_triple_loop]),
    "nvfp4_strided_groups": ([(nvfp4, "dequant_nvfp4", _dequant_nvfp4_variant(strided=True))],
                             [lambda: tn.test_single_column_spike_picks_its_code_and_group_scale(47)]),
    "nvfp4_block_scale_dropped": ([(nvfp4, "dequant_nvfp4", _dequant_nvfp4_variant(no_scale=True))],
                                  [tn.test_matches_exact_rational_triple_loop]),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, monkeypatch):
    patches, pins = MUTATIONS[name]
    for mod, attr, fn in patches:
        monkeypatch.setattr(mod, attr, fn)
    assert any(_fails(p) for p in pins), f"planted mistake {name} went unnoticed"
