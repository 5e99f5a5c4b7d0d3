"""Dequantize-and-matmul in float64, and the output tolerance check.

Test infrastructure: see the package docstring.

The block-scaled GEMM computes y[m, n] = sum_k A[m, k] * W[n, k] with
A[m, k] = dec(q[m, k]) * s[m, k // 128] and W[n, k] = dec(qw[n, k]) * ws[n // 128, k // 128]
(model card "Nanbeige4.3-33B FP8", introduction: E4M3 weights in 128x128 blocks,
dynamic per-token group-128 activation scales).  Promoting partial sums once per
128-wide K block, sum_kb (s * ws) * sum_{k in kb} dec(q) dec(qw), is only a
reordering of the same sum, so the oracle computes the plain definition: both
operands are dequantized exactly in float64 (an E4M3 value times a float32 scale
has at most 4 + 24 significant bits) and multiplied with one float64 BLAS matmul.

The card disclaims bit-exact equality across GEMM geometry (section "Compatibility
and limitations"), so the GPU output, which is BF16, is accepted element-wise when
|y - ref| <= REL_TOL * |ref| + RMS_TOL * rms(ref), rms taken over all checked
elements of that output.
"""

import numpy as np

from .e4m3 import decode

GROUP = 128
REL_TOL = 4e-3
RMS_TOL = 1e-3


def dequant_act(q, s):
    """float64 [M, K] activations from codes q [M, K] and scales s [M, K/128]."""
    q = np.asarray(q, dtype=np.uint8)
    s = np.asarray(s, dtype=np.float32)
    M, K = q.shape
    if s.shape != (M, K // GROUP):
        raise ValueError("activation scale shape mismatch")
    a = decode(q).reshape(M, K // GROUP, GROUP)
    return (a * s.astype(np.float64)[:, :, None]).reshape(M, K)


def dequant_weight(qw, ws):
    """float64 [N, K] weights from codes qw [N, K] and block scales ws [N/128, K/128]."""
    qw = np.asarray(qw, dtype=np.uint8)
    ws = np.asarray(ws, dtype=np.float32)
    N, K = qw.shape
    if ws.shape != (N // GROUP, K // GROUP):
        raise ValueError("weight scale shape mismatch")
    w = decode(qw).reshape(N // GROUP, GROUP, K // GROUP, GROUP)
    return (w * ws.astype(np.float64)[:, None, :, None]).reshape(N, K)


def linear_ref(q, s, qw, ws, w_deq=None):
    """float64 [M, N] = dequant_act(q, s) @ dequant_weight(qw, ws).T.

    ``w_deq`` may pass a precomputed dequant_weight(qw, ws) to reuse it across calls.
    """
    a = dequant_act(q, s)
    w = dequant_weight(qw, ws) if w_deq is None else w_deq
    if a.shape[1] != w.shape[1]:
        raise ValueError("K mismatch")
    return a @ w.T


def bf16_bits_to_f64(bits):
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def check_tolerance(y, ref):
    """Element-wise acceptance of a GPU output against the float64 reference.

    y: BF16 bit patterns (uint16) or float values, same shape as ref.
    Returns a dict with ok, n_fail, worst (max of |y-ref| / bound), rms.
    """
    ref = np.asarray(ref, dtype=np.float64)
    y = np.asarray(y)
    yv = bf16_bits_to_f64(y) if y.dtype == np.uint16 else y.astype(np.float64)
    if yv.shape != ref.shape:
        raise ValueError("shape mismatch")
    if ref.size == 0:
        return {"ok": True, "n_fail": 0, "worst": 0.0, "rms": 0.0}
    rms = float(np.sqrt(np.mean(ref * ref)))
    bound = REL_TOL * np.abs(ref) + RMS_TOL * rms
    err = np.abs(yv - ref)
    bad = ~(err <= bound)                     # NaN in y counts as a failure
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(bound > 0, err / bound, np.where(err > 0, np.inf, 0.0))
    return {
        "ok": not bool(bad.any()),
        "n_fail": int(bad.sum()),
        "worst": float(np.max(np.where(np.isnan(ratio), np.inf, ratio))),
        "rms": rms,
    }
