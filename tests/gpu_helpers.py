"""Helpers shared by the GPU parity tests: move oracle inputs to the device,
run the library through the C ABI, and apply the tolerance bar."""

import numpy as np
import torch

import blockwise_scaled_fp8_amd as bfp8
import oracle

FINITE_CODES = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)


def say(*args):
    print("[case]", *args, flush=True)


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    return t.detach().cpu()


def f32(t):
    """16-bit torch tensor -> exact float32 numpy."""
    return t.detach().float().cpu().numpy()


def workspace(op, M, N, K):
    n = bfp8.bfp8_workspace_bytes(op, M, N, K)
    return None if n == 0 else torch.zeros(n, dtype=torch.uint8, device="cuda")


def run_w8a8(xq, xs, wq, ws, out_dtype, ws_buf=None):
    M, K = xq.shape
    N = wq.shape[0]
    y = torch.empty((M, N), dtype=out_dtype, device="cuda")
    if ws_buf is None:
        ws_buf = workspace(bfp8.OP_GEMM_W8A8_BLK128, M, N, K)
    bfp8.bfp8_gemm_w8a8_blk128(xq, xs, wq, ws, y, ws_buf)
    torch.cuda.synchronize()
    return y


def run_w8a16(x, wq, ws, out_dtype, ws_buf=None):
    M, K = x.shape
    N = wq.shape[0]
    y = torch.empty((M, N), dtype=out_dtype, device="cuda")
    if ws_buf is None:
        ws_buf = workspace(bfp8.OP_GEMM_W8A16_BLK128, M, N, K)
    bfp8.bfp8_gemm_w8a16_blk128(x, wq, ws, y, ws_buf)
    torch.cuda.synchronize()
    return y


def run_blk32(x, wq, e8, out_dtype, ws_buf=None):
    M, K = x.shape
    N = wq.shape[0]
    y = torch.empty((M, N), dtype=out_dtype, device="cuda")
    if ws_buf is None:
        ws_buf = workspace(bfp8.OP_GEMM_W8A16_BLK32_UE8M0, M, N, K)
    bfp8.bfp8_gemm_w8a16_blk32_ue8m0(x, wq, e8, y, ws_buf)
    torch.cuda.synchronize()
    return y


def assert_fp32_bar(y, y0, what):
    ok, e = oracle.check_gemm_fp32(y.float().cpu().numpy(), y0)
    assert ok, f"{what}: {e}"
    return e


def assert_16bit_bar(y16, y32, y0, fmt, what):
    """16-bit output: the per-element bar and bitwise RNE of the kernel's own fp32."""
    ok, e = oracle.check_gemm_16bit(f32(y16), y0, fmt)
    assert ok, f"{what} ({fmt}): {e}"
    rne = y32.to(y16.dtype)
    assert torch.equal(rne.view(torch.int16), y16.view(torch.int16)), f"{what}: 16-bit output != RNE(fp32 output)"
    return e
