"""Seeded synthetic inputs for the W8A8 FP8 block-scaled linear.

This module holds no quantization or GEMM arithmetic: it only draws BF16 tensors.
Both sides of a parity check (the HIP path and the CPU oracle) receive the same
arrays from here; neither side produces the other's inputs.

Random numbers come from numpy's counter-based Philox4x32-10 bit generator
(Salmon et al., "Parallel random numbers: as easy as 1, 2, 3", SC'11).  Every
row of every tensor has its own stream, keyed by (seed, tensor id, row), so any
single row can be regenerated without drawing the rest of the tensor, and the
result does not depend on how the work is split across threads.  A float32
sample from the standard normal is scaled in float32 and rounded once to BF16
with round-to-nearest-even.

Workloads (the sizes are those of the serving model the pages describe: hidden
7168, 56 query and 8 KV heads of dimension 128, MLP width 8192, a draft block of
8 tokens and a 3 x 7168 -> 7168 feature-fusion projection):

  tiny           M=4,     K=512,   N=384    x ~ N(0,1),       W ~ N(0, 0.02)
  decode_qkv     M=1,     K=7168,  N=9216   x ~ N(0,1) with 72 outlier channels x20
  spec_mlp_gu    M=8,     K=7168,  N=16384  x ~ N(0,1);  N = [gate 8192 | up 8192]
  spec_mlp_down  M=8,     K=8192,  N=7168   input = SiLU(gate)*up of the gate/up output
  prefill_oproj  M=8191,  K=7168,  N=7168   as decode_qkv, plus 8 all-zero tokens
  fusion_fc      M=32768, K=21504, N=7168   x ~ N(0, s^2), s = 1, 2, 4 per 7168 segment;
                                            W ~ N(0, 0.01)

"N(0, 0.02)" is read as standard deviation 0.02.  "1% of channels" of K=7168 is 72
channels, chosen once per tensor by a seeded permutation and shared by all
tokens; "0.1% of tokens" of M=8191 is 8 rows set to +0.0.
"""

from .gen import (  # noqa: F401
    TID_X,
    TID_W,
    TID_OUTLIER,
    TID_ZERO,
    TID_ROWS,
    TID_GU,
    TID_W_DOWN,
    TID_GAMMA,
    TID_W4,
    TID_W4_SCALE,
    f32_to_bf16_bits,
    normal_rows,
    bf16_normal,
    uniform_bytes,
    choose,
    sample_rows,
)
from .workloads import WORKLOADS, Workload, make_activation, make_weight, activation_rows  # noqa: F401
from .w4a16 import W4A16_WORKLOADS, W4A16Workload, w4a16_activation_rows, w4a16_weight  # noqa: F401
