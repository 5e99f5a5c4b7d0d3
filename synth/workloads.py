"""The five synthetic workloads, as (shape, distribution) recipes."""

from dataclasses import dataclass, field

import numpy as np

from .gen import TID_OUTLIER, TID_W, TID_W_DOWN, TID_X, TID_ZERO, bf16_normal, choose, f32_to_bf16_bits, normal_rows


@dataclass(frozen=True)
class Workload:
    name: str
    M: int
    K: int
    N: int
    w_sigma: float
    x_kind: str                 # "normal" | "outliers" | "segments"
    outlier_frac: float = 0.0   # fraction of K channels scaled by outlier_mult
    outlier_mult: float = 20.0
    zero_token_frac: float = 0.0
    segments: tuple = ()        # per-segment sigma for x_kind == "segments"
    w_tid: int = TID_W
    seed: int = 0
    sampled_rows: int = 0       # 0: check every row; else seeded rows per check
    notes: str = field(default="", compare=False)

    @property
    def n_outliers(self):
        return int(round(self.outlier_frac * self.K))

    @property
    def n_zero_tokens(self):
        return int(round(self.zero_token_frac * self.M))

    def outlier_channels(self):
        return choose(self.K, self.n_outliers, self.seed, TID_OUTLIER) if self.n_outliers else np.zeros(0, np.int64)

    def zero_tokens(self):
        return choose(self.M, self.n_zero_tokens, self.seed, TID_ZERO) if self.n_zero_tokens else np.zeros(0, np.int64)

    def col_scale(self):
        s = np.ones(self.K, dtype=np.float32)
        if self.x_kind == "segments":
            seg = self.K // len(self.segments)
            for i, sig in enumerate(self.segments):
                s[i * seg:(i + 1) * seg] = np.float32(sig)
        if self.n_outliers:
            s[self.outlier_channels()] *= np.float32(self.outlier_mult)
        return s

    # Algorithmic work of one linear on this shape.
    def gemm_bytes(self):
        M, K, N = self.M, self.K, self.N
        return N * K + 4 * (N // 128) * (K // 128) + M * K + 4 * M * (K // 128) + 2 * M * N

    def gemm_flops(self):
        return 2 * self.M * self.N * self.K

    def quant_bytes(self):
        M, K = self.M, self.K
        return 2 * M * K + M * K + 4 * M * (K // 128)


WORKLOADS = {
    "tiny": Workload("tiny", 4, 512, 384, 0.02, "normal"),
    "decode_qkv": Workload("decode_qkv", 1, 7168, 9216, 0.02, "outliers", outlier_frac=0.01),
    "spec_mlp_gu": Workload("spec_mlp_gu", 8, 7168, 16384, 0.02, "normal"),
    "spec_mlp_down": Workload("spec_mlp_down", 8, 8192, 7168, 0.02, "silu", w_tid=TID_W_DOWN),
    "prefill_oproj": Workload("prefill_oproj", 8191, 7168, 7168, 0.02, "outliers",
                              outlier_frac=0.01, zero_token_frac=0.001, sampled_rows=256),
    "fusion_fc": Workload("fusion_fc", 32768, 21504, 7168, 0.01, "segments",
                          segments=(1.0, 2.0, 4.0), sampled_rows=256),
}


def activation_rows(wl, rows):
    """uint16 BF16 activations of the given rows of ``wl`` ([len(rows), K])."""
    if wl.x_kind == "silu":
        raise ValueError("the down projection's input comes from the gate/up output")
    rows = np.asarray(rows, dtype=np.int64).reshape(-1)
    x = normal_rows(rows, wl.K, wl.seed, TID_X, wl.col_scale())
    bits = f32_to_bf16_bits(x)
    if wl.n_zero_tokens:
        z = np.isin(rows, wl.zero_tokens())
        bits[z] = 0
    return bits


def make_activation(wl):
    return activation_rows(wl, np.arange(wl.M))


def make_weight(wl):
    """uint16 BF16 weights [N, K] ~ N(0, w_sigma^2)."""
    return bf16_normal(wl.N, wl.K, wl.w_sigma, wl.seed, wl.w_tid)
