"""Dynamic per-token group-128 activation quantizer, 128x128 block weight quantizer,
and the SiLU(gate)*up glue that feeds the down projection.

Test infrastructure: see the package docstring.

Scheme (model card "Nanbeige4.3-33B FP8", introduction and "Recipe and
calibration"): weights are E4M3 with one scale per 128x128 block from "standard
minmax" quantization; activations get dynamic scales per token and per group of
128 consecutive K elements.  The card fixes neither the scale dtype, the scale
formula beyond "minmax", the rounding of the quotient, nor the handling of an
all-zero group.  The readings taken here:

  * a scale is float32 and equals fl32(amax / 448): symmetric min/max gives
    max(|min|, |max|) = amax, mapped onto the largest finite E4M3 value 448;
  * each element is divided by its scale in float32 (one IEEE division,
    round-to-nearest-even, subnormals kept) and the quotient is encoded to E4M3
    with round-to-nearest-even, saturating at +-448;
  * an all-zero group has scale +0.0 and all codes 0x00;
  * NaN or infinite input is outside the contract and raises.

The model runs in BF16 (its serving command passes --dtype bfloat16, section
"Serving"), so the quantizer's input is BF16, and the SiLU(gate)*up product that
feeds the down projection is rounded to BF16 before it is re-quantized.
"""

import numpy as np

from .e4m3 import encode_rne_sat

GROUP = 128
E4M3_MAX = np.float32(448.0)


def bf16_bits_to_f32(bits):
    """BF16 bit patterns (uint16) to float32 values (exact widening)."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def f64_to_bf16_bits(h):
    """Round float64 values to BF16 once, nearest-even, and return the bit patterns.

    BF16 keeps 8 significant bits; its smallest quantum (subnormals) is 2^-133.
    A value h = m * 2^e with 0.5 <= |m| < 1 has the quantum 2^(max(e, -125) - 8).
    Scaling by a power of two and np.rint (ties to even) are exact in float64, so
    the result is the correctly rounded BF16 value, which float32 then holds
    exactly.
    """
    h = np.asarray(h, dtype=np.float64)
    if not np.isfinite(h).all():
        raise ValueError("BF16 rounding: non-finite value")
    _, e = np.frexp(h)
    e = np.maximum(e, -125)
    quantum_exp = (e - 8).astype(np.int64)
    r = np.ldexp(np.rint(np.ldexp(h, -quantum_exp)), quantum_exp)
    if (np.abs(r) >= 2.0 ** 128).any():
        raise ValueError("BF16 rounding: overflow")
    bits = (r.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    return bits


def _quant_groups(x, axes):
    """Quantize float32 ``x`` whose scale groups are reduced over ``axes``.

    Returns (codes uint8 with x's shape, scales float32 with ``axes`` reduced).
    """
    if not np.isfinite(x).all():
        raise ValueError("quantizer input must be finite")
    amax = np.max(np.abs(x), axis=axes, keepdims=True)       # exact, float32
    s = (amax / E4M3_MAX).astype(np.float32)                 # fl32(amax/448)
    zero = s == 0
    with np.errstate(divide="ignore", invalid="ignore"):
        v = (x / np.where(zero, np.float32(1), s)).astype(np.float32)
    v = np.clip(v, -E4M3_MAX, E4M3_MAX)
    q = encode_rne_sat(v)
    q = np.where(np.broadcast_to(zero, q.shape), np.uint8(0), q).astype(np.uint8)
    return q, np.squeeze(s, axis=axes).astype(np.float32)


def quant_act(x_bits):
    """Per-token, group-128 activation quantization.

    x_bits: uint16 [M, K] BF16 bit patterns, K a multiple of 128.
    Returns q uint8 [M, K] (E4M3 codes) and s float32 [M, K/128], where group g of
    row m covers columns [128 g, 128 g + 128).
    """
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    M, K = x_bits.shape
    if K % GROUP:
        raise ValueError("K must be a multiple of 128")
    x = bf16_bits_to_f32(x_bits).reshape(M, K // GROUP, GROUP)
    q, s = _quant_groups(x, axes=(2,))
    return q.reshape(M, K), s.reshape(M, K // GROUP)


def quant_weight(w_bits):
    """128x128 block weight quantization ("standard minmax", data independent).

    w_bits: uint16 [N, K] BF16 bit patterns (row n is output channel n, K contiguous).
    Returns qw uint8 [N, K] and ws float32 [N/128, K/128]; block (i, j) covers rows
    [128 i, 128 i + 128) and columns [128 j, 128 j + 128).
    """
    w_bits = np.asarray(w_bits, dtype=np.uint16)
    N, K = w_bits.shape
    if N % GROUP or K % GROUP:
        raise ValueError("N and K must be multiples of 128")
    w = bf16_bits_to_f32(w_bits).reshape(N // GROUP, GROUP, K // GROUP, GROUP)
    q, s = _quant_groups(w, axes=(1, 3))
    return q.reshape(N, K), s.reshape(N // GROUP, K // GROUP)


def silu_mul_bf16(gu_bits):
    """h = BF16(silu(gate) * up) with gate = columns [0, I) and up = [I, 2I).

    gu_bits: uint16 [M, 2I] BF16 bit patterns (the fused gate/up projection output).
    silu(g) = g / (1 + exp(-g)).  The product is evaluated in float64 and rounded
    to BF16 once, i.e. h is the BF16 rounding of the real value silu(g)*u (up to
    float64 error, 2^-40 of a BF16 half-ulp).
    """
    gu_bits = np.asarray(gu_bits, dtype=np.uint16)
    M, two_i = gu_bits.shape
    if two_i % 2:
        raise ValueError("gate/up width must be even")
    half = two_i // 2
    gu = bf16_bits_to_f32(gu_bits).astype(np.float64)
    if not np.isfinite(gu).all():
        raise ValueError("gate/up input must be finite")
    g, u = gu[:, :half], gu[:, half:]
    with np.errstate(over="ignore"):
        silu = g / (1.0 + np.exp(-g))
    return f64_to_bf16_bits(silu * u)


def silu_mul_quant(gu_bits):
    """Down-projection input: quant_act(silu_mul_bf16(gu))."""
    return quant_act(silu_mul_bf16(gu_bits))
