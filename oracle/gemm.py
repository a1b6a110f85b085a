"""Block-scaled products — oracle, test infrastructure only.

All three return Y[M, N] = X . W^T as float64 (weights stored [N, K],
K contiguous).  Rounding to a 16-bit output type is not done here: the parity
tests compare the GPU's fp32 accumulation with this float64 result and check
its 16-bit outputs against the round-to-nearest-even of its own fp32 result.

W8A8, 128x128 weight tiles and 1x128 activation groups
([ADA] "The starting point" and "The fix"; [ARC] "What this adds"):
    for each 128-wide K block kb:
        P[m, n] = sum_{k in kb} D[xq[m, k]] * D[wq[n, k]]
        Y[m, n] += P[m, n] * xs[m, kb] * ws[n // 128, kb]
  The weight-scale row is chosen per output column n (n // 128), not per tile
  of the GPU grid ([ADA] "The fix", the latent-bug paragraph).
  P is exact in float64 in any summation order: every product is a multiple
  of 2^-18 below 448^2 < 2^18 in magnitude, so any partial sum over 128 terms
  is an integer multiple of 2^-18 below 2^25 and fits in 43 bits.  That is why
  a library matmul may form P.  The promotion Y += P * (xs * ws) is the only
  rounding step; xs * ws is exact in float64 (two 24-bit significands).

W8A16, 128x128 weight tiles, 16-bit activations ([ARC] "What this adds"):
    Y[m, n] = sum_kb ws[n // 128, kb] * sum_{k in kb} x[m, k] * D[wq[n, k]]

W8A16, 32x32 tiles with power-of-two (UE8M0) scales ([SM70] "How it works",
"Exactness"): the byte E of tile (n // 32, k // 32) stands for 2^(E - 127);
    Y[m, n] = sum_k x[m, k] * (D[wq[n, k]] * 2^(E[n // 32, k // 32] - 127))
  Each scaled weight D * 2^e is a single float64 exactly.
"""

import numpy as np

from .e4m3 import e4m3_decode

BLK128 = 128
BLK32 = 32


def _check_codes(q):
    d = e4m3_decode(q)
    if np.isnan(d).any():
        raise ValueError("E4M3 NaN code (0x7F / 0xFF) in operand")
    return d


def gemm_w8a8_blk128(xq, xs, wq, ws):
    """W8A8 blockwise product.  xq [M,K] u8, xs [M,K/128] f32, wq [N,K] u8,
    ws [ceil(N/128), K/128] f32.  K must be a multiple of 128."""
    xq, wq = np.asarray(xq, np.uint8), np.asarray(wq, np.uint8)
    xs, ws = np.asarray(xs, np.float32), np.asarray(ws, np.float32)
    M, K = xq.shape
    N = wq.shape[0]
    assert wq.shape[1] == K and K % BLK128 == 0
    KB = K // BLK128
    assert xs.shape == (M, KB) and ws.shape == (-(-N // BLK128), KB)
    xd, wd = _check_codes(xq), _check_codes(wq)
    nb_of_col = np.arange(N) // BLK128
    y = np.zeros((M, N), dtype=np.float64)
    for kb in range(KB):
        ks = slice(kb * BLK128, (kb + 1) * BLK128)
        P = xd[:, ks] @ wd[:, ks].T                      # exact, see module doc
        scale = xs[:, kb].astype(np.float64)[:, None] * ws[nb_of_col, kb].astype(np.float64)[None, :]
        y += P * scale
    return y


def gemm_w8a16_blk128(x, wq, ws):
    """W8A16 blockwise product.  x [M,K] 16-bit values given as f32,
    wq [N,K] u8, ws [ceil(N/128), K/128] f32.  K must be a multiple of 128."""
    x = np.asarray(x, np.float32).astype(np.float64)
    wq, ws = np.asarray(wq, np.uint8), np.asarray(ws, np.float32)
    M, K = x.shape
    N = wq.shape[0]
    assert wq.shape[1] == K and K % BLK128 == 0
    KB = K // BLK128
    assert ws.shape == (-(-N // BLK128), KB)
    wd = _check_codes(wq)
    nb_of_col = np.arange(N) // BLK128
    y = np.zeros((M, N), dtype=np.float64)
    for kb in range(KB):
        ks = slice(kb * BLK128, (kb + 1) * BLK128)
        y += (x[:, ks] @ wd[:, ks].T) * ws[nb_of_col, kb].astype(np.float64)[None, :]
    return y


def gemm_w8a16_blk32_ue8m0(x, wq, e8m0):
    """W8A16 32x32 power-of-two product.  x [M,K] 16-bit values given as f32,
    wq [N,K] u8, e8m0 [N/32, K/32] u8 (2^(E-127)).  N, K multiples of 32."""
    x = np.asarray(x, np.float32).astype(np.float64)
    wq, e8m0 = np.asarray(wq, np.uint8), np.asarray(e8m0, np.uint8)
    M, K = x.shape
    N = wq.shape[0]
    assert wq.shape[1] == K and K % BLK32 == 0 and N % BLK32 == 0
    assert e8m0.shape == (N // BLK32, K // BLK32)
    scale = np.exp2(e8m0.astype(np.float64) - 127.0)
    w_scaled = _check_codes(wq) * np.repeat(np.repeat(scale, BLK32, axis=0), BLK32, axis=1)
    return x @ w_scaled.T
