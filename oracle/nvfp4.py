"""NVFP4 weight-only (W4A16) linear: E2M1 weight codes in groups of 16 along K, one
E4M3 scale per group, one float32 global scale per tensor, BF16 activations.

Test infrastructure: see the package docstring.

The "Nanbeige4.3-33B-NVFP4-A16" model card (the paragraph on the base revision and
calibration) fixes the scheme: FP4 E2M1 weights in groups of 16 with E4M3 block
scales and a global weight scale, activations left in BF16 (no activation
quantization), serialized in the loader convention that keeps packed FP4 values
and block scales and stores the global scale as a multiplier (its export step turns
the calibrator's global-scale reciprocals around).  The card does not print the
arithmetic; the reading taken here is the plain dequantize-then-multiply one:

    W[n, k] = e2m1(code[n, k]) * e4m3(bs[n, k // 16]) * g
    y[m, n] = sum_k x[m, k] * W[n, k]

computed in float64 (every W[n, k] is exact there: 2 + 4 + 24 significant bits)
with one float64 BLAS matmul; the GPU output is BF16 and is accepted with the
tolerance of ``linear.check_tolerance``.

E2M1 is the 4-bit element format of the OCP Microscaling (MX) specification: 1 sign
bit, 2 exponent bits with bias 1, 1 mantissa bit; exponent field 0 holds the
subnormal m * 0.5; there is no infinity or NaN, so the 16 codes are the values
+-{0, 0.5, 1, 1.5, 2, 3, 4, 6}.

Packing (the card says only "packed FP4 values"; the reading taken): two codes per
byte along K, element 2j in the low nibble and element 2j + 1 in the high nibble of
byte j of the row, so a row of K codes is K / 2 bytes.  Block scales are E4M3 bytes
[N, K / 16], row-major.
"""

import numpy as np

from .e4m3 import decode as e4m3_decode
from .quant import bf16_bits_to_f32

GROUP16 = 16


def e2m1_decode_table():
    """float64[16]: the value of every E2M1 code (OCP MX element format)."""
    vals = np.empty(16, dtype=np.float64)
    for code in range(16):
        sign = -1.0 if code & 0x8 else 1.0
        e = (code >> 1) & 0x3
        m = code & 0x1
        if e == 0:
            vals[code] = sign * m * 0.5
        else:
            vals[code] = sign * (1.0 + m / 2.0) * 2.0 ** (e - 1)
    return vals


_E2M1 = e2m1_decode_table()


def unpack_fp4(packed):
    """uint8 [N, K] codes from packed bytes [N, K / 2] (low nibble = even element)."""
    p = np.asarray(packed, dtype=np.uint8)
    if p.ndim != 2:
        raise ValueError("packed weights must be [N, K/2]")
    N, H = p.shape
    codes = np.empty((N, 2 * H), dtype=np.uint8)
    codes[:, 0::2] = p & 0x0F
    codes[:, 1::2] = p >> 4
    return codes


def dequant_nvfp4(packed, bs, g):
    """float64 [N, K] weights: e2m1(code) * e4m3(bs[n, k // 16]) * g."""
    codes = unpack_fp4(packed)
    N, K = codes.shape
    bs = np.asarray(bs, dtype=np.uint8)
    if K % GROUP16 or bs.shape != (N, K // GROUP16):
        raise ValueError("block scales must be [N, K/16]")
    sc = e4m3_decode(bs)
    if np.isnan(sc).any():
        raise ValueError("block scale NaN codes are outside the oracle's contract")
    gv = float(np.float32(g))
    if not np.isfinite(gv):
        raise ValueError("global scale must be finite")
    w = _E2M1[codes].reshape(N, K // GROUP16, GROUP16) * sc[:, :, None]
    return w.reshape(N, K) * gv


def linear_w4a16_ref(x_bits, packed, bs, g, w_deq=None):
    """float64 [M, N] = x @ dequant_nvfp4(packed, bs, g).T with BF16 x [M, K].

    ``w_deq`` may pass a precomputed dequant_nvfp4(packed, bs, g) to reuse it.
    """
    x = bf16_bits_to_f32(np.asarray(x_bits, dtype=np.uint16)).astype(np.float64)
    if x.ndim != 2:
        raise ValueError("x must be [M, K]")
    w = dequant_nvfp4(packed, bs, g) if w_deq is None else w_deq
    if x.shape[1] != w.shape[1]:
        raise ValueError("K mismatch")
    if not np.isfinite(x).all():
        raise ValueError("activations must be finite")
    return x @ w.T
