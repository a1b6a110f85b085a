"""CPU oracle for the blockwise-scaled FP8 GEMM — TEST INFRASTRUCTURE ONLY.

This package is the slow, plain, obviously-correct definition of what the GPU
library computes.  It is used only by ``tests/``, by ``__graft_entry__.smoke()``
and by the ``cpu_baseline`` leg of ``bench.py``.  The product path (the HIP
library and its Python binding) never imports it, and it imports nothing from
the product path: the two share no code, tables or constants.

Everything is numpy in float64 unless a step's precision is fixed by the
method (the activation/weight scale and the quotient x/s are IEEE fp32, as the
quantiser produces fp32 scales and rounds the scaled value once before
encoding).

Pages cited (by title and section):
  [ADA]   "Blockwise FP8 on Ada GPUs, part 2: my kernel was correct and 4x too
          slow" (amankarki.hashnode.dev)
  [ARC]   "perf(ArcKernels): blockwise-FP8 GEMM on tensor cores, scale promoted
          per 128-K" (GitHub pull request, including the "Route-2 handover"
          comment)
  [SM70]  "SM70 FP8 block-32 kernels (PLI Labs)" (Hugging Face model card)
  [3090]  "FP8 / NVFP4 の weight-only 推論で RTX 3090 が失っているものは無い"
          (minamism.com)

Modules:
  e4m3    decode (closed form) and round-to-nearest-even saturating encode
  quant   1x128 activation quantiser and 128x128 weight quantiser
  gemm    W8A8 blk128, W8A16 blk128 and W8A16 blk32-UE8M0 products
  ue8m0   load-time validation of power-of-two block scales
  dequant load-time blockwise dequantisation (the fallback for refused layers)
  compare the tolerance bar used by the parity tests

Every function is pinned by tests in ``tests/test_oracle_*.py`` against facts
the pages or mathematics fix (bitwise identities, brute force, exact rational
arithmetic, library special cases); the tolerance bar in ``compare`` is pinned
by hand-computed error measures, arrays just inside and just outside each
bound, and half-ulps checked against the 16-bit formats' bit patterns
(``tests/test_oracle_compare.py``).  Planted mistakes in copies of these
functions make a pin fail (``tests/test_oracle_mutations.py``).  No function
is "parity unpinned".
"""

from .e4m3 import e4m3_decode, e4m3_encode, E4M3_MAX, E4M3_NAN_CODES
from .quant import quantize_act_1x128, quantize_weight_128x128
from .gemm import gemm_w8a8_blk128, gemm_w8a16_blk128, gemm_w8a16_blk32_ue8m0
from .ue8m0 import prepare_blk32_ue8m0, Refusal
from .dequant import dequantize_weight, round_bf16, round_f16
from .compare import gemm_error, check_gemm_fp32, check_gemm_16bit

__all__ = [
    "e4m3_decode", "e4m3_encode", "E4M3_MAX", "E4M3_NAN_CODES",
    "quantize_act_1x128", "quantize_weight_128x128",
    "gemm_w8a8_blk128", "gemm_w8a16_blk128", "gemm_w8a16_blk32_ue8m0",
    "prepare_blk32_ue8m0", "Refusal",
    "dequantize_weight", "round_bf16", "round_f16",
    "gemm_error", "check_gemm_fp32", "check_gemm_16bit",
]
