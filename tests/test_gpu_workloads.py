"""GPU parity at the workloads' full sizes, in the launch configuration the bench uses.

Quantization: bit-exact codes and scales (every row, except fusion_fc: 256 seeded
rows).  GEMM: the tolerance on every element of the checked rows (all rows for the
decode shapes; prefill_oproj: 256 seeded rows, its 8 zero tokens and the ragged
last row; fusion_fc: 256 seeded rows).  The speculative MLP runs as a chain: gate/up
GEMM (tolerance), SiLU(gate)*up re-quantized from the GPU's own gate/up output
(bit-exact), down GEMM on those codes (tolerance)."""

import numpy as np
import pytest
import torch

import fp8_block_scaled_amd as fb
import oracle
import synth
from synth import WORKLOADS
from tests.gpu_util import assert_bits_equal, banner, dev_bf16, host_f32, host_u16, host_u8

pytestmark = pytest.mark.gpu


def checked_rows(wl):
    if not wl.sampled_rows:
        return np.arange(wl.M)
    rows = synth.sample_rows(wl.M, wl.sampled_rows, wl.seed)
    extra = np.concatenate([wl.zero_tokens(), [wl.M - 1]])
    return np.unique(np.concatenate([rows, extra])).astype(np.int64)


def run_linear_workload(name):
    wl = WORKLOADS[name]
    banner(f"workload {name}: generate")
    x = synth.make_activation(wl)
    w = synth.make_weight(wl)
    banner(f"workload {name}: GPU M={wl.M} K={wl.K} N={wl.N}")
    qg, sg = fb.quant_act(dev_bf16(x))
    qwg, wsg = fb.quant_weight(dev_bf16(w))
    yg = fb.block_linear(qg, sg, qwg, wsg)
    torch.cuda.synchronize()
    rows = checked_rows(wl)
    rows_t = torch.from_numpy(rows).cuda()
    q_rows, s_rows = host_u8(qg[rows_t]), host_f32(sg[rows_t])
    y_rows = host_u16(yg[rows_t])
    qw_h, ws_h = host_u8(qwg), host_f32(wsg)
    del qg, sg, qwg, wsg, yg
    banner(f"workload {name}: oracle on {len(rows)} rows")
    qo, so = oracle.quant_act(x[rows])
    assert_bits_equal(s_rows, so, f"{name} activation scales")
    assert_bits_equal(q_rows, qo, f"{name} activation codes")
    qwo, wso = oracle.quant_weight(w)
    assert_bits_equal(ws_h, wso, f"{name} weight scales")
    assert_bits_equal(qw_h, qwo, f"{name} weight codes")
    ref = oracle.linear_ref(qo, so, qwo, wso)
    res = oracle.check_tolerance(y_rows, ref)
    print(f"[parity] {name}: {res}", flush=True)
    assert res["ok"], f"{name}: {res}"
    if wl.n_zero_tokens:
        z = np.isin(rows, wl.zero_tokens())
        assert np.all(y_rows[z] == 0)
    return res


@pytest.mark.parametrize("name", ["tiny", "decode_qkv", "spec_mlp_gu", "prefill_oproj", "fusion_fc"])
def test_linear_workload(name):
    run_linear_workload(name)


# Standard deviation of the gate/up output for x ~ N(0,1), W ~ N(0, 0.02^2), K = 7168:
# sqrt(7168) * 0.02 = 1.69.
GU_SIGMA = 1.7


def test_spec_mlp_down_stage():
    """The down projection at full size on a shared seeded gate/up tensor: both sides
    apply SiLU(gate)*up and re-quantize (bit-exact), then the GEMM (tolerance)."""
    gu_wl, dn_wl = WORKLOADS["spec_mlp_gu"], WORKLOADS["spec_mlp_down"]
    gu = synth.bf16_normal(gu_wl.M, gu_wl.N, GU_SIGMA, gu_wl.seed, synth.TID_GU)
    w_dn = synth.make_weight(dn_wl)
    banner("workload spec_mlp_down: GPU")
    q2, s2 = fb.silu_mul_quant(dev_bf16(gu))
    qw2, ws2 = fb.quant_weight(dev_bf16(w_dn))
    y = fb.block_linear(q2, s2, qw2, ws2)
    torch.cuda.synchronize()
    banner("workload spec_mlp_down: oracle")
    hq, hs = oracle.silu_mul_quant(gu)
    assert_bits_equal(host_f32(s2), hs, "down input scales")
    assert_bits_equal(host_u8(q2), hq, "down input codes")
    qw2o, ws2o = oracle.quant_weight(w_dn)
    assert_bits_equal(host_u8(qw2), qw2o, "down weight codes")
    res = oracle.check_tolerance(host_u16(y), oracle.linear_ref(hq, hs, qw2o, ws2o))
    print(f"[parity] spec_mlp_down: {res}", flush=True)
    assert res["ok"], f"down: {res}"


def test_spec_mlp_chain():
    """x -> gate/up -> SiLU(gate)*up re-quantized -> down, element by element.

    The gate/up output is checked against the oracle within the GEMM tolerance.  The
    re-quantization is then checked bit-exact on the GPU's own gate/up output (both
    sides quantize the same BF16 tensor), and the down GEMM within the tolerance
    against the oracle's dequantize-and-matmul of those same codes: every stage of
    the chain is held to its own element-wise bar, with no stage's input taken from
    the other side's rounding."""
    gu_wl, dn_wl = WORKLOADS["spec_mlp_gu"], WORKLOADS["spec_mlp_down"]
    banner("workload spec_mlp chain: generate")
    x = synth.make_activation(gu_wl)
    w_gu = synth.make_weight(gu_wl)
    w_dn = synth.make_weight(dn_wl)
    banner("workload spec_mlp chain: GPU")
    q, s = fb.quant_act(dev_bf16(x))
    qw1, ws1 = fb.quant_weight(dev_bf16(w_gu))
    qw2, ws2 = fb.quant_weight(dev_bf16(w_dn))
    gu = fb.block_linear(q, s, qw1, ws1)
    q2, s2 = fb.silu_mul_quant(gu)
    y = fb.block_linear(q2, s2, qw2, ws2)
    torch.cuda.synchronize()
    gu_h, y_h, q2_h, s2_h = host_u16(gu), host_u16(y), host_u8(q2), host_f32(s2)
    banner("workload spec_mlp chain: oracle")
    qo, so = oracle.quant_act(x)
    assert_bits_equal(host_u8(q), qo, "gate/up input codes")
    qw1o, ws1o = oracle.quant_weight(w_gu)
    qw2o, ws2o = oracle.quant_weight(w_dn)
    r1 = oracle.check_tolerance(gu_h, oracle.linear_ref(qo, so, qw1o, ws1o))
    print(f"[parity] spec_mlp chain gate/up: {r1}", flush=True)
    assert r1["ok"], f"gate/up: {r1}"
    h_q, h_s = oracle.silu_mul_quant(gu_h)
    assert_bits_equal(s2_h, h_s, "down input scales (from the GPU's gate/up output)")
    assert_bits_equal(q2_h, h_q, "down input codes (from the GPU's gate/up output)")
    r2 = oracle.check_tolerance(y_h, oracle.linear_ref(h_q, h_s, qw2o, ws2o))
    print(f"[parity] spec_mlp chain down: {r2}", flush=True)
    assert r2["ok"], f"down: {r2}"
