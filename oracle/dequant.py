"""Blockwise weight dequantisation (load-time fallback) — oracle, test
infrastructure only.

[SM70] "Exactness": the block-32 packer refuses a layer whose 32x32 scales are
not powers of two inside [2^-14, 2^7], and such a layer is served by
dequantising its weights once, when they are loaded.  [ARC] "Route-2
handover" names dequantising per step as the pattern to avoid, so this is a
load-time conversion, not part of a GEMM.  The pages fix only "the E4M3 value
times its block scale"; the reading taken here:

    w[n, k] = RN_out( fl32( E4M3(wq[n, k]) * s[n // B, k // B] ) )

with B = 32 or 128, the product rounded once to fp32 (IEEE multiply), then
rounded to nearest even to the output type (bf16 or fp16; fp32 output is the
product itself).  Scales are row-major [ceil(N/B), ceil(K/B)]; a ragged last
block covers the remaining rows or columns only.  NaN codes give NaN.
"""

import numpy as np

from .e4m3 import e4m3_decode


def dequantize_weight(wq, scales, block):
    """fp32 weights fl32(E4M3(wq) * s) of wq [N, K] u8 with fp32 block scales.

    Returns a float32 array [N, K].
    """
    wq = np.asarray(wq, dtype=np.uint8)
    scales = np.asarray(scales, dtype=np.float32)
    N, K = wq.shape
    assert block in (32, 128)
    assert scales.shape == (-(-N // block), -(-K // block)), scales.shape
    out = np.empty((N, K), dtype=np.float32)
    for nb in range(scales.shape[0]):
        for kb in range(scales.shape[1]):
            rows = slice(nb * block, min(N, (nb + 1) * block))
            cols = slice(kb * block, min(K, (kb + 1) * block))
            d = e4m3_decode(wq[rows, cols]).astype(np.float32)    # exact: at most 4 significant bits
            out[rows, cols] = d * scales[nb, kb]                   # one IEEE fp32 rounding
    return out


def round_bf16(x):
    """Nearest-even bf16 value of each fp32 value, returned as fp32.

    Written out on the fp32 bit pattern: add 0x7FFF plus the lowest kept bit,
    then drop the low 16 bits (NaN stays NaN).
    """
    x = np.asarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    out = r.astype(np.uint32).view(np.float32)
    return np.where(np.isnan(x), np.float32(np.nan), out)


def round_f16(x):
    """Nearest-even fp16 value of each fp32 value (numpy's IEEE conversion;
    magnitudes past the fp16 range become infinities)."""
    with np.errstate(over="ignore"):
        return np.asarray(x, dtype=np.float32).astype(np.float16)
