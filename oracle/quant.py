"""Block quantisers — oracle, test infrastructure only.

Activations: one fp32 scale per token per 128 consecutive K values ("1x128
groups"), the layout [ADA] "The starting point" describes for vLLM's
checkpoints and [ARC] "Route-2 handover" item 2 gives as scales of shape
[M, ceil(K/128)].  Weights: one fp32 scale per 128x128 tile of W[N, K]
([ADA] "The starting point"; [ARC] "What this adds", the [N/128, K/128]
block scale).

Per group (or tile) the pages fix only "amax, scale, FP8 codes".  The reading
taken here, written out so that both sides can take the integer decision in
the same precision:
    amax = max |x| over the group (bf16/fp16 values widened exactly to fp32)
    s    = fl32(amax / 448)             correctly rounded fp32 division
    q_k  = enc(fl32(x_k / s))           one fp32 division per element, then
                                        round-to-nearest-even E4M3, saturating
    amax == 0  ->  s = 0 and every code 0x00.
A ragged last group (K not a multiple of 128) covers the remaining columns
only; so does a ragged last weight tile in either direction.
Scales are stored row-major: xs[m, g] and ws[nb, kb].
"""

import numpy as np

from .e4m3 import e4m3_encode, E4M3_MAX

GROUP = 128


def _quantize_group(vals):
    """Codes and fp32 scale of one group, given as an fp32 numpy array."""
    vals = np.asarray(vals, dtype=np.float32)
    amax = np.float32(np.max(np.abs(vals))) if vals.size else np.float32(0.0)
    if amax == 0.0:
        return np.zeros(vals.shape, dtype=np.uint8), np.float32(0.0)
    s = np.float32(amax / np.float32(E4M3_MAX))          # IEEE fp32 division
    scaled = (vals / s).astype(np.float32)               # IEEE fp32 division
    return e4m3_encode(scaled), s


def quantize_act_1x128(x):
    """1x128 activation quantisation.

    x: [M, K] array of fp32 values that are exactly bf16 or fp16 values.
    Returns xq uint8 [M, K] (E4M3 codes) and xs float32 [M, ceil(K/128)].
    """
    x = np.asarray(x, dtype=np.float32)
    M, K = x.shape
    G = -(-K // GROUP)
    xq = np.zeros((M, K), dtype=np.uint8)
    xs = np.zeros((M, G), dtype=np.float32)
    for m in range(M):
        for g in range(G):
            lo, hi = g * GROUP, min(K, (g + 1) * GROUP)
            xq[m, lo:hi], xs[m, g] = _quantize_group(x[m, lo:hi])
    return xq, xs


def quantize_weight_128x128(w):
    """128x128 weight quantisation.

    w: [N, K] array of fp32 values that are exactly bf16 values.
    Returns wq uint8 [N, K] and ws float32 [ceil(N/128), ceil(K/128)].
    """
    w = np.asarray(w, dtype=np.float32)
    N, K = w.shape
    NB, KB = -(-N // GROUP), -(-K // GROUP)
    wq = np.zeros((N, K), dtype=np.uint8)
    ws = np.zeros((NB, KB), dtype=np.float32)
    for nb in range(NB):
        for kb in range(KB):
            rows = slice(nb * GROUP, min(N, (nb + 1) * GROUP))
            cols = slice(kb * GROUP, min(K, (kb + 1) * GROUP))
            wq[rows, cols], ws[nb, kb] = _quantize_group(w[rows, cols])
    return wq, ws
