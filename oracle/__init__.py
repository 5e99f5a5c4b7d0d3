"""CPU oracle for the W8A8 FP8 block-scaled linear -- TEST INFRASTRUCTURE ONLY.

This package is the plain, slow, obviously-correct reference that the HIP path is
checked against.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it.  The product package
``fp8_block_scaled_amd`` never imports it, and it imports nothing from the product
package: the two share no code, tables, constants or helpers.

What it computes follows the "Nanbeige4.3-33B FP8" model card (ProCreations),
introduction and section "Recipe and calibration": W8A8 FP8 with E4M3 weights in
128x128 blocks and dynamic per-token, group-128 activation scales (scheme
FP8_BLOCK, "standard minmax" weight quantization).  The E4M3 bit format itself is
the OCP 8-bit Floating Point Specification (OFP8), E4M3 encoding.  The weight-only
NVFP4 variant (``nvfp4``) follows the "Nanbeige4.3-33B-NVFP4-A16" model card and the
E2M1 element format of the OCP Microscaling specification.

Floating point: scales and quotients are float32 (the precision the method fixes
for them, see ``quant``); dequantization and the matmul are float64 (``linear``).

Modules
  e4m3    -- decode table from the format definition; nearest-even encoder with
             saturation (table + midpoint search).
  quant   -- per-token group-128 activation quantizer, 128x128 block weight
             quantizer, SiLU(gate)*up in float64 rounded once to BF16.
  rmsnorm -- RMSNorm in float64 rounded once to BF16, then the quantizer.
  linear  -- dequantize-and-matmul in float64 and the output tolerance check.
  nvfp4   -- the NVFP4 weight-only variant: E2M1 codes, E4M3 group-16 scales and a
             global scale against BF16 activations, in float64.

Parity pins (tests/test_oracle_*.py) tie every function to something other than
itself: closed-form code values, the torch CPU float8_e4m3fn cast, an independent
bit-manipulation encoder, exact rational arithmetic (fractions / decimal) on
small inputs and invariants of the scheme.
"""

from .e4m3 import decode_table, decode, encode_rne_sat  # noqa: F401
from .quant import (  # noqa: F401
    bf16_bits_to_f32,
    f64_to_bf16_bits,
    quant_act,
    quant_weight,
    silu_mul_bf16,
    silu_mul_quant,
)
from .rmsnorm import rmsnorm_bf16, rmsnorm_quant  # noqa: F401
from .linear import (  # noqa: F401
    dequant_act,
    dequant_weight,
    linear_ref,
    check_tolerance,
    REL_TOL,
    RMS_TOL,
)
from .nvfp4 import (  # noqa: F401
    e2m1_decode_table,
    unpack_fp4,
    dequant_nvfp4,
    linear_w4a16_ref,
)
