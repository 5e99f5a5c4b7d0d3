"""RMSNorm of a BF16 hidden state, rounded once to BF16, then the per-token group-128
quantizer: the input of the FP8 q/k/v projection.

Test infrastructure: see the package docstring.

The pages place an RMSNorm right before the projections the FP8 linear serves: the
"Nanbeige4.3-33B DMS sidecar" card ("Format and hipEngine compatibility") reads its
input at the normalized stage after the post-attention RMSNorm and before the q
projection, and the "Nanbeige4.3-33B DFlash2" card's architecture table lists an
RMS epsilon of 1e-5 and a hidden RMSNorm after the feature-fusion projection.
Neither card gives the arithmetic.  The reading taken here is the textbook one:

    h[m, k] = x[m, k] / sqrt(mean_k x[m, k]^2 + eps) * gamma[k]

with BF16 x and gamma, evaluated in float64 and rounded to BF16 once (no
intermediate BF16 rounding of the normalized value), eps a float32 value.
"""

import numpy as np

from .quant import bf16_bits_to_f32, f64_to_bf16_bits, quant_act


def rmsnorm_bf16(x_bits, gamma_bits, eps):
    """h = BF16(x / sqrt(mean(x^2) + eps) * gamma) per row, in float64, rounded once.

    x_bits: uint16 [M, K] BF16 bit patterns; gamma_bits: uint16 [K]; eps: float32 > 0
    (taken exactly, widened to float64).
    """
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    gamma_bits = np.asarray(gamma_bits, dtype=np.uint16)
    if x_bits.ndim != 2 or gamma_bits.shape != (x_bits.shape[1],):
        raise ValueError("x must be [M, K] and gamma [K]")
    eps = float(np.float32(eps))
    if not eps > 0:
        raise ValueError("eps must be positive")
    x = bf16_bits_to_f32(x_bits).astype(np.float64)
    g = bf16_bits_to_f32(gamma_bits).astype(np.float64)
    if not (np.isfinite(x).all() and np.isfinite(g).all()):
        raise ValueError("RMSNorm input must be finite")
    ms = np.mean(x * x, axis=1, keepdims=True)
    r = 1.0 / np.sqrt(ms + eps)
    return f64_to_bf16_bits((x * r) * g)


def rmsnorm_quant(x_bits, gamma_bits, eps):
    """Projection input: quant_act(rmsnorm_bf16(x, gamma, eps))."""
    return quant_act(rmsnorm_bf16(x_bits, gamma_bits, eps))
