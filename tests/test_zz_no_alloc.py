"""The allocation-free W8A8 entry point (bfp8_gemm_w8a8_blk128_noalloc, for
callers that cannot allocate) against the workspace entry point
bfp8_gemm_w8a8_blk128, through the C ABI: bit-identical outputs on two calls
in a row, the second with a smaller input (so the second call finds the
first call's contents in the shared scratch), for plans that split K (the
scratch holds counters and partial tiles) and plans that need no workspace;
fp32 output also against the float64 oracle's bar."""

import numpy as np
import pytest
import torch

import blockwise_scaled_fp8_amd as bfp8
from blockwise_scaled_fp8_amd import inputs
import oracle
from tests.gpu_helpers import say, dev, f32, workspace, assert_fp32_bar
from tests.cases import variant, W8A8

pytestmark = pytest.mark.gpu


def _operands(M, N, K, wid):
    x = inputs.activations(M, K, workload=wid, stream=0, outliers=True)
    w = inputs.weights_bf16(N, K, workload=wid, stream=1)
    xq, xs = oracle.quantize_act_1x128(f32(x))
    wq, ws = oracle.quantize_weight_128x128(f32(w))
    return xq, xs, wq, ws


def _both(xq, xs, wq, ws, out_dtype):
    M, K = xq.shape
    N = wq.shape[0]
    y_ref = torch.empty((M, N), dtype=out_dtype, device="cuda")
    bfp8.bfp8_gemm_w8a8_blk128(xq, xs, wq, ws, y_ref, workspace(bfp8.OP_GEMM_W8A8_BLK128, M, N, K))
    y = torch.full((M, N), float("nan"), dtype=out_dtype, device="cuda")
    bfp8.bfp8_gemm_w8a8_blk128_noalloc(xq, xs, wq, ws, y)
    torch.cuda.synchronize()
    return y, y_ref


@pytest.mark.parametrize("first,second", [
    ((400, 2048, 8192), (100, 1024, 8192)),     # 128x128 split 4, then 64x128 split 8
    ((200, 2048, 4224), (16, 512, 12288)),      # 64x128 split 4, then the streaming kernel split over K
    ((128, 4096, 4096), (1, 1024, 4096)),       # no workspace: all-token kernel, then one token
    ((24, 1024, 12288), (5, 1024, 12288)),      # all-token kernel with K split 4 ways, twice (counters re-armed)
    ((32, 4096, 12288), (20, 2064, 12288)),     # 32-row all-token tiles split two ways, then fewer of them
])
def test_noalloc_matches_workspace_call(gpu_lib, first, second):
    assert np.prod(second) < np.prod(first)
    for i, (M, N, K) in enumerate((first, second)):
        say("noalloc", i, f"M={M} N={N} K={K}", variant(W8A8, M, N, K))
        xq, xs, wq, ws = _operands(M, N, K, 1000 + 7 * i + M)
        d = [dev(a) for a in (xq, xs, wq, ws)]
        for out in (torch.float32, torch.bfloat16):
            y, y_ref = _both(*d, out)
            view = torch.int32 if out == torch.float32 else torch.int16
            assert torch.equal(y.view(view), y_ref.view(view)), (M, N, K, out)
            if out == torch.float32:
                assert_fp32_bar(y, oracle.gemm_w8a8_blk128(xq, xs, wq, ws), f"noalloc M={M} N={N} K={K}")


def test_noalloc_repeated_calls_re_arm(gpu_lib):
    """Three calls in a row on one split-K plan give the same bits (the
    counters the kernel leaves behind are cleared for the next call)."""
    M, N, K = 65, 1024, 8192
    assert "/split" in variant(W8A8, M, N, K)
    d = [dev(a) for a in _operands(M, N, K, 1100)]
    ys = []
    for _ in range(3):
        y = torch.empty((M, N), dtype=torch.float32, device="cuda")
        bfp8.bfp8_gemm_w8a8_blk128_noalloc(*d, y)
        ys.append(y)
    torch.cuda.synchronize()
    assert torch.equal(ys[0].view(torch.int32), ys[1].view(torch.int32))
    assert torch.equal(ys[0].view(torch.int32), ys[2].view(torch.int32))
