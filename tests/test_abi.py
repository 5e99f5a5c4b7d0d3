"""The C ABI library loads, exports every symbol include/fp8bs.h declares, and rejects
bad arguments on the host before any GPU work (no compute calls are made here)."""

import ctypes
import os
import re

import pytest

from fp8_block_scaled_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp8bs.h")

OK, ENULL, ESHAPE, EALIGN, EDEV, EHIP, EWS, EVAL = 0, -1, -2, -3, -4, -5, -6, -7
# Fake, never-dereferenced addresses: validation must reject before using them.
A16, A16b, A16c, A16d, A16e = 0x10000, 0x20000, 0x30000, 0x40000, 0x50000


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w]*\s*\*?\s*((?:fp8|nvfp4)\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def L():
    return _lib.lib()


def test_header_declares_the_boundary():
    names = declared_functions()
    assert {"fp8_quant_act", "fp8_block_linear", "nvfp4_w4a16_linear"} <= set(names)
    assert set(names) == set(_lib.SIGNATURES), names


def test_every_declared_symbol_is_exported(L):
    for name in declared_functions():
        assert hasattr(L, name), name


def test_version_and_status_strings(L):
    assert L.fp8bs_abi_version() == 10400
    for st in (OK, ENULL, ESHAPE, EALIGN, EDEV, EHIP, EWS, EVAL):
        assert L.fp8bs_status_string(st)
    assert b"unknown" in L.fp8bs_status_string(12345)


def test_quant_act_validation(L):
    assert L.fp8_quant_act(None, A16, A16b, 4, 128, None) == ENULL
    assert L.fp8_quant_act(A16, A16b, A16c, 4, 200, None) == ESHAPE
    assert L.fp8_quant_act(A16, A16b, A16c, -1, 128, None) == ESHAPE
    assert L.fp8_quant_act(A16, A16b, A16c, 1 << 40, 1 << 40, None) == ESHAPE
    assert L.fp8_quant_act(A16 + 2, A16b, A16c, 4, 128, None) == EALIGN
    assert L.fp8_quant_act(A16, A16b + 8, A16c, 4, 128, None) == EALIGN
    assert L.fp8_quant_act(A16, A16b, A16c + 2, 4, 128, None) == EALIGN
    assert L.fp8_quant_act(None, None, None, 0, 128, None) == OK      # empty: no-op


def test_weight_and_silu_validation(L):
    assert L.fp8_quant_weight(A16, A16b, A16c, 100, 128, None) == ESHAPE
    assert L.fp8_quant_weight(A16, A16b, A16c, 128, 100, None) == ESHAPE
    assert L.fp8_quant_weight(None, A16b, A16c, 128, 128, None) == ENULL
    assert L.fp8_silu_mul_quant(A16, A16b, A16c, 2, 100, None) == ESHAPE
    assert L.fp8_silu_mul_quant(A16, None, A16c, 2, 128, None) == ENULL
    assert L.fp8_silu_mul_quant(A16, A16b, A16c, 0, 128, None) == OK


def test_rmsnorm_quant_validation(L):
    f = L.fp8_rmsnorm_quant
    assert f(A16, A16b, 1e-5, A16c, A16d, 4, 200, None) == ESHAPE
    assert f(A16, None, 1e-5, A16c, A16d, 4, 128, None) == ENULL
    assert f(A16, A16b + 2, 1e-5, A16c, A16d, 4, 128, None) == EALIGN
    assert f(A16, A16b, 0.0, A16c, A16d, 4, 128, None) == EVAL
    assert f(A16, A16b, -1e-5, A16c, A16d, 4, 128, None) == EVAL
    assert f(A16, A16b, float("nan"), A16c, A16d, 4, 128, None) == EVAL
    assert f(A16, A16b, float("inf"), A16c, A16d, 4, 128, None) == EVAL
    assert f(None, None, 1e-5, None, None, 0, 128, None) == OK        # empty: no-op


def test_block_linear_validation(L):
    f = L.fp8_block_linear
    assert f(A16, A16b, A16c, A16d, A16e, 4, 100, 128, None, 0, None) == ESHAPE
    assert f(A16, A16b, A16c, A16d, A16e, 4, 128, 100, None, 0, None) == ESHAPE
    assert f(A16, A16b, A16c, A16d, A16e, 4, 128, 0, None, 0, None) == ESHAPE
    assert f(A16, A16b, A16c, A16d, A16e, -4, 128, 128, None, 0, None) == ESHAPE
    assert f(None, A16b, A16c, A16d, A16e, 4, 128, 128, None, 0, None) == ENULL
    assert f(A16, A16b, A16c, A16d, None, 4, 128, 128, None, 0, None) == ENULL
    assert f(A16 + 4, A16b, A16c, A16d, A16e, 4, 128, 128, None, 0, None) == EALIGN
    assert f(A16, A16b + 1, A16c, A16d, A16e, 4, 128, 128, None, 0, None) == EALIGN
    assert f(A16, A16b, A16c, A16d, A16e + 8, 4, 128, 128, None, 0, None) == EALIGN
    assert f(A16, A16b, A16c, A16d, A16e, 4, 128, 128, A16 + 16, 4096, None) == EWS
    assert f(None, None, None, None, None, 0, 128, 128, None, 0, None) == OK     # M == 0
    assert f(None, None, None, None, None, 4, 0, 128, None, 0, None) == OK       # N == 0


def test_block_linear_noalloc_validation(L):
    f = L.fp8_block_linear_noalloc
    assert f(A16, A16b, A16c, A16d, A16e, 4, 100, 128, None) == ESHAPE
    assert f(A16, A16b, A16c, A16d, A16e, 4, 128, 0, None) == ESHAPE
    assert f(A16, A16b, A16c, A16d, A16e, -4, 128, 128, None) == ESHAPE
    assert f(None, A16b, A16c, A16d, A16e, 4, 128, 128, None) == ENULL
    assert f(A16, A16b, A16c, A16d, None, 4, 128, 128, None) == ENULL
    assert f(A16 + 4, A16b, A16c, A16d, A16e, 4, 128, 128, None) == EALIGN
    assert f(A16, A16b, A16c, A16d + 2, A16e, 4, 128, 128, None) == EALIGN
    assert f(None, None, None, None, None, 0, 128, 128, None) == OK     # M == 0
    # The largest split-K workspace any valid shape asks for fits the static scratch
    # (32 MiB: at most 256 / t ways of t 128 x 256 tiles, so 256 * 256 * 4 * 128 bytes).
    for shape in ((33, 7168, 7168), (128, 7168, 7168), (100, 1024, 8192), (128, 16384, 7168), (200, 128, 8192),
                  (256, 7168, 7168), (384, 7168, 7168), (512, 7168, 7168), (256, 16384, 7168), (512, 1024, 8192)):
        assert 0 < L.fp8_block_linear_workspace_size(*shape) <= 32 << 20, shape


def test_nvfp4_linear_validation(L):
    f = L.nvfp4_w4a16_linear
    A = (A16, A16b, A16c)
    assert f(*A, 1.0, A16d, 4, 100, 128, None, 0, None) == ESHAPE
    assert f(*A, 1.0, A16d, 4, 128, 112, None, 0, None) == ESHAPE
    assert f(*A, 1.0, A16d, 4, 128, 0, None, 0, None) == ESHAPE
    assert f(*A, 1.0, A16d, -1, 128, 128, None, 0, None) == ESHAPE
    assert f(*A, 1.0, A16d, 1 << 32, 128, 128, None, 0, None) == ESHAPE      # 32-bit token rows
    assert f(*A, float("nan"), A16d, 4, 128, 128, None, 0, None) == EVAL
    assert f(*A, float("inf"), A16d, 4, 128, 128, None, 0, None) == EVAL
    assert f(None, A16b, A16c, 1.0, A16d, 4, 128, 128, None, 0, None) == ENULL
    assert f(A16, A16b, None, 1.0, A16d, 4, 128, 128, None, 0, None) == ENULL
    assert f(A16 + 2, A16b, A16c, 1.0, A16d, 4, 128, 128, None, 0, None) == EALIGN
    assert f(A16, A16b + 8, A16c, 1.0, A16d, 4, 128, 128, None, 0, None) == EALIGN
    assert f(A16, A16b, A16c + 8, 1.0, A16d, 4, 128, 128, None, 0, None) == EALIGN
    assert f(A16, A16b, A16c, 1.0, A16d + 2, 4, 128, 128, None, 0, None) == EALIGN
    assert f(*A, 1.0, A16d, 4, 128, 128, A16e + 16, 4096, None) == EWS
    assert f(None, None, None, 1.0, None, 0, 128, 128, None, 0, None) == OK     # M == 0
    assert f(None, None, None, -2.5, None, 4, 0, 128, None, 0, None) == OK      # N == 0


def test_nvfp4_workspace_size_query(L):
    q = L.nvfp4_w4a16_workspace_size
    assert q(1, 9216, 7168) == 0 and q(16, 7168, 8192) == 0 and q(32, 7168, 7168) == 0    # decode / streaming
    assert q(64, 7168, 7168) == 8 * 64 * 7168 * 4                        # split-K tiles above 32 rows
    assert q(33, 7168, 7168) == 8 * 33 * 7168 * 4
    assert q(2048, 7168, 7168) == 0                                      # enough tiles without a split
    assert q(128, 16384, 7168) == 4 * 128 * 16384 * 4                     # 64 tiles: split 4
    assert q(100, 1024, 1152) == 8 * 100 * 1024 * 4                       # split capped at 8 ...
    assert q(100, 1024, 256) == 2 * 100 * 1024 * 4                        # ... and at half the K steps
    assert q(100, 1024, 128) == 0
    for bad in ((-1, 128, 128), (4, 100, 128), (4, 128, 0)):
        assert q(*bad) == 0


def test_valid_call_without_a_gpu_reports_a_hip_error_not_a_crash(L):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert L.fp8_quant_act(A16, A16b, A16c, 4, 128, None) in (EHIP, EDEV)


def test_workspace_size_query(L):
    for shape in ((8191, 7168, 7168), (4, 100, 128), (-1, 128, 128), (1, 9216, 7168), (8, 7168, 8192),
                  (24, 7168, 7168), (32, 7168, 7168), (2048, 7168, 7168)):
        assert L.fp8_block_linear_workspace_size(*shape) == 0
    assert L.fp8_block_linear_workspace_size(33, 7168, 7168) == 4 * 33 * 7168 * 4   # split-K above 32 rows
    # 56 tiles of 128 x 128: split 4 (256 / 56), FP32 [4][M][N]
    assert L.fp8_block_linear_workspace_size(128, 7168, 7168) == 4 * 128 * 7168 * 4
    # capped at 8 ways and at a quarter of the K blocks
    assert L.fp8_block_linear_workspace_size(100, 1024, 8192) == 8 * 100 * 1024 * 4
    assert L.fp8_block_linear_workspace_size(100, 1024, 1024) == 2 * 100 * 1024 * 4
    assert L.fp8_block_linear_workspace_size(100, 1024, 512) == 0


def test_nvfp4_binding_rejects_bad_tensors_before_any_gpu_call():
    import torch
    import fp8_block_scaled_amd as fb
    x = torch.zeros((2, 256), dtype=torch.bfloat16)
    w4 = torch.zeros((128, 128), dtype=torch.uint8)
    bs = torch.zeros((128, 16), dtype=torch.uint8)
    with pytest.raises(ValueError, match="GPU"):          # CPU tensors: no CPU path
        fb.nvfp4_linear(x, w4, bs, 1.0)
    with pytest.raises(TypeError):                        # not a tensor
        fb.nvfp4_linear([[0.0] * 256] * 2, w4, bs, 1.0)


def test_binding_rejects_wrong_outputs_before_any_gpu_call():
    """Caller-supplied outputs (q, s, out) and operands are checked for dtype, exact
    shape and contiguity before any pointer reaches the library: a wrong-sized output
    would let a kernel write past its allocation."""
    import torch
    import fp8_block_scaled_amd as fb
    bf = torch.bfloat16
    x = torch.zeros((4, 256), dtype=bf)
    q_ok = torch.zeros((4, 256), dtype=torch.uint8)
    s_ok = torch.zeros((4, 2), dtype=torch.float32)
    with pytest.raises(ValueError, match="shape"):
        fb.quant_act(x, q=torch.zeros((4, 128), dtype=torch.uint8), s=s_ok)
    with pytest.raises(ValueError, match="shape"):
        fb.quant_act(x, q=q_ok, s=torch.zeros((4, 1), dtype=torch.float32))
    with pytest.raises(TypeError):
        fb.quant_act(x, q=q_ok, s=torch.zeros((4, 2), dtype=torch.float64))
    with pytest.raises(ValueError, match="contiguous"):
        fb.quant_act(x, q=torch.zeros((256, 4), dtype=torch.uint8).t(), s=s_ok)
    with pytest.raises(ValueError, match="multiple of 128"):
        fb.quant_act(torch.zeros((4, 200), dtype=bf))
    gu = torch.zeros((4, 512), dtype=bf)
    with pytest.raises(ValueError, match="shape"):
        fb.silu_mul_quant(gu, q=torch.zeros((4, 512), dtype=torch.uint8), s=s_ok)
    with pytest.raises(ValueError, match="shape"):
        fb.rmsnorm_quant(x, torch.zeros((128,), dtype=bf), 1e-5)
    with pytest.raises(ValueError, match="shape"):
        fb.rmsnorm_quant(x, torch.zeros((256,), dtype=bf), 1e-5, q=q_ok, s=torch.zeros((2, 4), dtype=torch.float32))
    qw = torch.zeros((128, 256), dtype=torch.uint8)
    ws = torch.zeros((1, 2), dtype=torch.float32)
    with pytest.raises(ValueError, match="shape"):
        fb.block_linear(q_ok, s_ok, qw, ws, out=torch.zeros((4, 256), dtype=bf))
    with pytest.raises(ValueError, match="shape"):
        fb.block_linear(q_ok, torch.zeros((2, 4), dtype=torch.float32), qw, ws)
    with pytest.raises(ValueError, match="shape"):
        fb.block_linear(q_ok, s_ok, qw, torch.zeros((2, 1), dtype=torch.float32))
    with pytest.raises(TypeError):
        fb.block_linear(q_ok, s_ok, qw, ws, out=torch.zeros((4, 128), dtype=torch.float32))
    with pytest.raises(TypeError):
        fb.block_linear(q_ok, s_ok, qw, ws, workspace=torch.zeros(1024, dtype=torch.float32))
    w4 = torch.zeros((128, 128), dtype=torch.uint8)
    bs = torch.zeros((128, 16), dtype=torch.uint8)
    with pytest.raises(ValueError, match="shape"):
        fb.nvfp4_linear(x, w4, bs, 1.0, out=torch.zeros((4, 256), dtype=bf))
    with pytest.raises(ValueError, match="shape"):
        fb.nvfp4_linear(x, w4, torch.zeros((128, 8), dtype=torch.uint8), 1.0)
    # Correct shapes on the CPU: rejected for the device, not for a shape.
    with pytest.raises(ValueError, match="GPU"):
        fb.block_linear(q_ok, s_ok, qw, ws, out=torch.zeros((4, 128), dtype=bf))
