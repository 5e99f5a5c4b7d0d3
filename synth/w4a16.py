"""Synthetic workloads of the NVFP4 weight-only (W4A16) linear.

The packed 4-bit weight codes are uniform random bytes (every code equally likely,
both nibbles of a byte independent), the per-group scale codes are uniform on
the byte range [scale_lo, scale_hi] (positive E4M3 values 32 ... 240 with the
defaults), and the global scale is a fixed float32 chosen so that the weights have
a root mean square of about 0.02, like the BF16 weights of the FP8 workloads.  No
quantizer runs here: the kernel's work does not depend on how the codes were
chosen.  Activations are BF16 N(0, 1) with 1% outlier channels x20 (the decode
projections' recipe).

Shapes are those of the serving model (hidden 7168, q/k/v 9216, gate/up 2 x 8192,
down 8192 -> 7168) in the regimes the NVFP4 card measures: single-stream decode
(M = 1), a 128-stream decode step (M = 128) and a 2048-token prefill chunk.
"""

from dataclasses import dataclass

import numpy as np

from .gen import TID_OUTLIER, TID_W4, TID_W4_SCALE, TID_X, choose, f32_to_bf16_bits, normal_rows, uniform_bytes


@dataclass(frozen=True)
class W4A16Workload:
    name: str
    M: int
    K: int
    N: int
    outlier_frac: float = 0.01
    outlier_mult: float = 20.0
    scale_lo: int = 0x60
    scale_hi: int = 0x77
    g: float = 5.5e-5
    seed: int = 0
    sampled_rows: int = 0

    @property
    def n_outliers(self):
        return int(round(self.outlier_frac * self.K))

    def col_scale(self):
        s = np.ones(self.K, dtype=np.float32)
        if self.n_outliers:
            s[choose(self.K, self.n_outliers, self.seed, TID_OUTLIER)] *= np.float32(self.outlier_mult)
        return s

    # Algorithmic work of one linear: packed codes, group scales, x and y.
    def gemm_bytes(self):
        M, K, N = self.M, self.K, self.N
        return N * K // 2 + N * K // 16 + 2 * M * K + 2 * M * N

    def gemm_flops(self):
        return 2 * self.M * self.N * self.K


W4A16_WORKLOADS = {
    "w4a16_tiny": W4A16Workload("w4a16_tiny", 5, 512, 384),
    "w4a16_decode_qkv": W4A16Workload("w4a16_decode_qkv", 1, 7168, 9216),
    "w4a16_decode_gu": W4A16Workload("w4a16_decode_gu", 1, 7168, 16384),
    "w4a16_decode_down": W4A16Workload("w4a16_decode_down", 1, 8192, 7168),
    "w4a16_batch128_gu": W4A16Workload("w4a16_batch128_gu", 128, 7168, 16384, sampled_rows=32),
    "w4a16_prefill_chunk": W4A16Workload("w4a16_prefill_chunk", 2048, 7168, 7168, sampled_rows=256),
}


def w4a16_activation_rows(wl, rows):
    """uint16 BF16 activations of the given rows of ``wl`` ([len(rows), K])."""
    rows = np.asarray(rows, dtype=np.int64).reshape(-1)
    return f32_to_bf16_bits(normal_rows(rows, wl.K, wl.seed, TID_X, wl.col_scale()))


def w4a16_weight(wl):
    """(packed uint8 [N, K/2], group scale codes uint8 [N, K/16], float32 g)."""
    packed = uniform_bytes(wl.N, wl.K // 2, 0, 255, wl.seed, TID_W4)
    scales = uniform_bytes(wl.N, wl.K // 16, wl.scale_lo, wl.scale_hi, wl.seed, TID_W4_SCALE)
    return packed, scales, np.float32(wl.g)
