"""fp8_block_linear_noalloc (the entry point that allocates nothing) against
fp8_block_linear with a workspace, through the C ABI: bitwise-equal outputs (same
schedule, same summation order) and both within the tolerance of the oracle, on
consecutive calls -- a 3-way split-K call on 128 x 256 tiles, a 4-way split-K call on
128 x 128 tiles, then a smaller 2-way split-K call that finds the earlier calls'
partial sums in the shared scratch, then a decode shape."""

import numpy as np
import pytest
import torch

import fp8_block_scaled_amd as fb
import oracle
import synth
from fp8_block_scaled_amd import _lib
from tests.gpu_util import banner, dev_bf16, host_f32, host_u16, host_u8

pytestmark = pytest.mark.gpu

# (M, N, K, split-K ways of the schedule on a 256-CU device)
CASES = [(384, 7168, 7168, 3), (128, 7168, 7168, 4), (48, 2048, 1024, 2), (4, 1024, 512, 0)]


def _inputs(M, N, K, seed):
    x = synth.bf16_normal(M, K, 1.0, seed, synth.TID_X)
    w = synth.bf16_normal(N, K, 0.02, seed, synth.TID_W)
    return x, w


def test_noalloc_matches_workspace_call_on_consecutive_calls():
    L = _lib.lib()
    for i, (M, N, K, split) in enumerate(CASES):
        banner(f"fp8_block_linear_noalloc call {i}: M={M} N={N} K={K} split={split}")
        x, w = _inputs(M, N, K, seed=100 + i)
        q, s = fb.quant_act(dev_bf16(x))
        qw, ws = fb.quant_weight(dev_bf16(w))
        need = fb.workspace_size(M, N, K)
        assert need == split * M * N * 4
        assert need <= 32 << 20                          # FP8BS_NOALLOC_SCRATCH_BYTES
        work = torch.empty(max(need, 256), dtype=torch.uint8, device="cuda")
        y_ws = fb.block_linear(q, s, qw, ws, workspace=work)
        y = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
        rc = L.fp8_block_linear_noalloc(q.data_ptr(), s.data_ptr(), qw.data_ptr(), ws.data_ptr(), y.data_ptr(),
                                        M, N, K, torch.cuda.current_stream().cuda_stream)
        assert rc == 0, L.fp8bs_status_string(rc)
        torch.cuda.synchronize()
        yb, yw = host_u16(y), host_u16(y_ws)
        assert np.array_equal(yb, yw), f"call {i}: {int(np.sum(yb != yw))} outputs differ from the workspace call"
        qo, so = oracle.quant_act(x)
        qwo, wso = oracle.quant_weight(w)
        assert np.array_equal(host_u8(q), qo) and np.array_equal(host_f32(s).view(np.uint32), so.view(np.uint32))
        res = oracle.check_tolerance(yb, oracle.linear_ref(qo, so, qwo, wso))
        assert res["ok"], f"call {i}: {res}"
