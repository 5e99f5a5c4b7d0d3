"""The C ABI from a plain C program (tests/c_abi/abi_roundtrip.c, built by build()):
no Python binding and no torch in the process.  It quantizes its own BF16 inputs and
runs the GEMM with the workspace the size query asks for; the outputs are checked
here against the oracle (quantization bit-exact, GEMM within the tolerance)."""

import os
import subprocess

import numpy as np
import pytest

import oracle
from tests.gpu_util import assert_bits_equal, banner

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BIN = os.path.join(ROOT, "tests", "c_abi", "abi_roundtrip")

pytestmark = pytest.mark.gpu


def read(path):
    with open(path, "rb") as f:
        M, N, K = np.frombuffer(f.read(24), dtype=np.int64)
        M, N, K = int(M), int(N), int(K)

        def take(dtype, n):
            return np.frombuffer(f.read(np.dtype(dtype).itemsize * n), dtype=dtype)
        x = take(np.uint16, M * K).reshape(M, K)
        w = take(np.uint16, N * K).reshape(N, K)
        q = take(np.uint8, M * K).reshape(M, K)
        s = take(np.float32, M * K // 128).reshape(M, K // 128)
        qw = take(np.uint8, N * K).reshape(N, K)
        ws = take(np.float32, N * K // 16384).reshape(N // 128, K // 128)
        y = take(np.uint16, M * N).reshape(M, N)
    return x, w, q, s, qw, ws, y


@pytest.mark.parametrize("M,N,K", [(1, 1024, 2048), (8, 384, 512), (40, 2048, 1024), (128, 2048, 2048),
                                   (300, 1024, 1152)])
def test_c_caller(M, N, K, tmp_path):
    assert os.path.exists(BIN), "tests/c_abi/abi_roundtrip is missing: run __graft_entry__.build()"
    out = tmp_path / "out.bin"
    banner(f"C caller M={M} N={N} K={K}")
    p = subprocess.run([BIN, str(M), str(N), str(K), str(M + N + K), str(out)], capture_output=True, text=True,
                       timeout=60)
    assert p.returncode == 0, p.stdout + p.stderr
    x, w, q, s, qw, ws, y = read(out)
    qo, so = oracle.quant_act(x)
    assert_bits_equal(s, so, "C caller: activation scales")
    assert_bits_equal(q, qo, "C caller: activation codes")
    qwo, wso = oracle.quant_weight(w)
    assert_bits_equal(ws, wso, "C caller: weight scales")
    assert_bits_equal(qw, qwo, "C caller: weight codes")
    res = oracle.check_tolerance(y, oracle.linear_ref(q, s, qw, ws))
    assert res["ok"], res
