"""Blockwise-scaled FP8 GEMM for AMD Instinct MI355X (gfx950).

The computation lives in libbfp8.so (HIP kernels behind the C ABI declared in
include/bfp8.h).  This package is the thin Python side: ``_lib`` marshals
torch tensors into the C calls (same names), and the helpers below only
allocate outputs and workspaces with torch before calling them.
"""

import torch

from ._lib import (  # noqa: F401
    BFP8_BF16, BFP8_F16, BFP8_F32, Bfp8Error, LIB_PATH, SIGNATURES, STATUS_NAMES,
    OP_QUANT_ACT_1X128, OP_QUANT_WEIGHT_128X128, OP_GEMM_W8A8_BLK128, OP_GEMM_W8A16_BLK128,
    OP_GEMM_W8A16_BLK32_UE8M0, OP_QUANT_GEMM_W8A8_BLK128,
    load, bfp8_quantize_act_1x128, bfp8_quantize_weight_128x128, bfp8_dequantize_weight,
    bfp8_gemm_w8a8_blk128, bfp8_gemm_w8a8_blk128_noalloc, bfp8_quant_gemm_w8a8_blk128, NOALLOC_SCRATCH_BYTES,
    bfp8_gemm_w8a16_blk128, bfp8_gemm_w8a16_blk32_ue8m0, bfp8_prepare_blk32_ue8m0,
    bfp8_workspace_bytes, bfp8_get_limits, bfp8_get_plan, bfp8_kernel_name, bfp8_status_string,
)


def make_workspace(op, M, N, K, device="cuda"):
    """A zero-filled workspace of the size the op needs (None when it needs
    none).  Zero-filled once; every call leaves it ready for the next.  Do not
    share one workspace between calls that may run at the same time."""
    n = bfp8_workspace_bytes(op, M, N, K)
    return None if n == 0 else torch.zeros(n, dtype=torch.uint8, device=device)


def quantize_act(x):
    """x [M, K] bf16/fp16 on the GPU -> (xq uint8 [M, K], xs float32 [M, ceil(K/128)])."""
    M, K = x.shape
    xq = torch.empty((M, K), dtype=torch.uint8, device=x.device)
    xs = torch.empty((M, (K + 127) // 128), dtype=torch.float32, device=x.device)
    bfp8_quantize_act_1x128(x, xq, xs)
    return xq, xs


def quantize_weight(w):
    """w [N, K] bf16/fp16 on the GPU -> (wq uint8 [N, K], ws float32 [ceil(N/128), ceil(K/128)])."""
    N, K = w.shape
    wq = torch.empty((N, K), dtype=torch.uint8, device=w.device)
    ws = torch.empty(((N + 127) // 128, (K + 127) // 128), dtype=torch.float32, device=w.device)
    bfp8_quantize_weight_128x128(w, wq, ws)
    return wq, ws


def dequantize_weight(wq, scales, block, out_dtype=torch.bfloat16):
    """wq [N, K] E4M3 codes with fp32 block scales (block 32 or 128) ->
    weights [N, K] in out_dtype (load-time fallback; see include/bfp8.h)."""
    w = torch.empty(wq.shape, dtype=out_dtype, device=wq.device)
    bfp8_dequantize_weight(wq, scales, block, w)
    return w


def gemm_w8a8(xq, xs, wq, ws, out_dtype=torch.bfloat16, workspace=None):
    M, N = xq.shape[0], wq.shape[0]
    y = torch.empty((M, N), dtype=out_dtype, device=xq.device)
    if workspace is None:
        workspace = make_workspace(OP_GEMM_W8A8_BLK128, M, N, xq.shape[1], xq.device)
    bfp8_gemm_w8a8_blk128(xq, xs, wq, ws, y, workspace)
    return y


def quant_gemm_w8a8(x, wq, ws, out_dtype=torch.bfloat16, workspace=None):
    """16-bit activations in: 1x128 quantisation and the W8A8 GEMM in one call."""
    M, N = x.shape[0], wq.shape[0]
    y = torch.empty((M, N), dtype=out_dtype, device=x.device)
    if workspace is None:
        workspace = make_workspace(OP_QUANT_GEMM_W8A8_BLK128, M, N, x.shape[1], x.device)
    bfp8_quant_gemm_w8a8_blk128(x, wq, ws, y, workspace)
    return y


def gemm_w8a16(x, wq, ws, out_dtype=None, workspace=None):
    M, N = x.shape[0], wq.shape[0]
    y = torch.empty((M, N), dtype=out_dtype or x.dtype, device=x.device)
    if workspace is None:
        workspace = make_workspace(OP_GEMM_W8A16_BLK128, M, N, x.shape[1], x.device)
    bfp8_gemm_w8a16_blk128(x, wq, ws, y, workspace)
    return y


def gemm_w8a16_blk32(x, wq, e8m0, out_dtype=torch.float16, workspace=None):
    M, N = x.shape[0], wq.shape[0]
    y = torch.empty((M, N), dtype=out_dtype, device=x.device)
    if workspace is None:
        workspace = make_workspace(OP_GEMM_W8A16_BLK32_UE8M0, M, N, x.shape[1], x.device)
    bfp8_gemm_w8a16_blk32_ue8m0(x, wq, e8m0, y, workspace)
    return y
