"""GPU parity at the longest K the calls accept (2^23, workload 5).

Every kernel family that can run there (streaming with in-kernel or staged
tokens, all-token, tiled, block-32) is launched on the whole problem, with K
split across workgroups as its plan says.  Its buffer offsets then reach
their largest values: weight and token rows 8 MiB apart, or 16 MiB for
16-bit tokens.  The oracle checks sampled outputs: the first and last token
rows against a few weight rows of the first scale row, or against the whole
first and last 32-row bands for block-32.
Each sampled output is a float64 sum over 65 536 scale blocks.  The bar is
the one every other parity test uses."""

import numpy as np
import pytest
import torch

import blockwise_scaled_fp8_amd as bfp8
from blockwise_scaled_fp8_amd import inputs
import oracle
from tests.gpu_helpers import say, f32, workspace, run_w8a8, run_w8a16, run_blk32, assert_fp32_bar, \
    assert_16bit_bar
from tests import cases
from tests.cases import expect, W8A8, QW8A8, W8A16, BLK32

pytestmark = pytest.mark.gpu

WID = 5


def _rows(n):
    """First and last row, and one inside the first 32-row band when there is room."""
    return sorted({0, min(5, n - 1), n - 1})


def _pick(y, rm, rn):
    return y[torch.tensor(rm, device=y.device)][:, torch.tensor(rn, device=y.device)]


def _codes_and_scales(M, N, K):
    xq = inputs.e4m3_codes(M, K, WID, 0)
    xs = inputs.block_scales(M, K // 128, WID, 1)
    wq = inputs.e4m3_codes(N, K, WID, 2)
    ws = inputs.block_scales((N + 127) // 128, K // 128, WID, 3)
    return xq, xs, wq, ws


@pytest.mark.parametrize("M,N,K,kernel", cases.W8A8_MAX_K)
def test_w8a8_longest_k(gpu_lib, M, N, K, kernel):
    say("w8a8 longest K", f"M={M} N={N} K={K}", kernel)
    expect(W8A8, M, N, K, kernel)
    assert N <= 128                                  # one weight-scale row: every sampled row uses ws[0]
    xq, xs, wq, ws = _codes_and_scales(M, N, K)
    d = [a.cuda() for a in (xq, xs, wq, ws)]
    y32 = run_w8a8(*d, torch.float32)
    y16 = run_w8a8(*d, torch.bfloat16)
    del d
    rm, rn = _rows(M), _rows(N)
    y0 = oracle.gemm_w8a8_blk128(xq[rm].numpy(), xs[rm].numpy(), wq[rn].numpy(), ws[:1].numpy())
    assert_fp32_bar(_pick(y32, rm, rn), y0, f"w8a8 M={M} N={N} K={K}")
    assert_16bit_bar(_pick(y16, rm, rn), _pick(y32, rm, rn), y0, "bf16", f"w8a8 M={M} N={N} K={K}")


@pytest.mark.parametrize("M,N,K,kernel", cases.QUANT_W8A8_MAX_K)
def test_quant_gemm_longest_k(gpu_lib, M, N, K, kernel):
    """The fused call at K = 2^23 is bit-identical to the quantiser followed by
    the codes call, its codes equal the oracle quantiser's, and sampled
    outputs meet the bar."""
    say("quant+w8a8 longest K", f"M={M} N={N} K={K}", kernel)
    expect(QW8A8, M, N, K, kernel)
    assert N <= 128
    x = inputs.activations(M, K, WID, stream=4)
    _, _, wq, ws = _codes_and_scales(1, N, K)
    xd, wqd, wsd = x.cuda(), wq.cuda(), ws.cuda()
    xq, xs = bfp8.quantize_act(xd)
    ref = run_w8a8(xq, xs, wqd, wsd, torch.float32)
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    bfp8.bfp8_quant_gemm_w8a8_blk128(xd, wqd, wsd, y, workspace(bfp8.OP_QUANT_GEMM_W8A8_BLK128, M, N, K))
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int32), ref.view(torch.int32))
    q0, s0 = oracle.quantize_act_1x128(f32(x))
    np.testing.assert_array_equal(xq.cpu().numpy(), q0)
    np.testing.assert_array_equal(xs.cpu().numpy(), s0)
    rn = _rows(N)
    y0 = oracle.gemm_w8a8_blk128(q0, s0, wq[rn].numpy(), ws[:1].numpy())
    assert_fp32_bar(_pick(y, list(range(M)), rn), y0, f"quant+w8a8 M={M} N={N} K={K}")


@pytest.mark.parametrize("M,N,K,kernel", cases.W8A16_MAX_K)
def test_w8a16_longest_k(gpu_lib, M, N, K, kernel):
    say("w8a16 longest K", f"M={M} N={N} K={K}", kernel)
    expect(W8A16, M, N, K, kernel)
    assert N <= 128
    x = inputs.activations(M, K, WID, stream=5)
    _, _, wq, ws = _codes_and_scales(1, N, K)
    xd, wqd, wsd = x.cuda(), wq.cuda(), ws.cuda()
    y32 = run_w8a16(xd, wqd, wsd, torch.float32)
    y16 = run_w8a16(xd, wqd, wsd, torch.bfloat16)
    del xd, wqd
    rm, rn = _rows(M), _rows(N)
    y0 = oracle.gemm_w8a16_blk128(f32(x[rm]), wq[rn].numpy(), ws[:1].numpy())
    assert_fp32_bar(_pick(y32, rm, rn), y0, f"w8a16 M={M} N={N} K={K}")
    assert_16bit_bar(_pick(y16, rm, rn), _pick(y32, rm, rn), y0, "bf16", f"w8a16 M={M} N={N} K={K}")


@pytest.mark.parametrize("M,N,K,kernel", cases.BLK32_MAX_K)
def test_blk32_longest_k(gpu_lib, M, N, K, kernel):
    say("blk32 longest K", f"M={M} N={N} K={K}", kernel)
    expect(BLK32, M, N, K, kernel)
    x = inputs.activations(M, K, WID, stream=6, dtype=torch.float16)
    wq = inputs.e4m3_codes(N, K, WID, 7).numpy()
    # exponents low enough that sums over 2^23 products stay well inside fp16
    s = inputs.block32_scales(N, K, WID, stream=8, lo=-14, hi=-8).numpy()
    st, e8, bad = oracle.prepare_blk32_ue8m0(wq, s)
    assert st == oracle.Refusal.OK, (st, bad)
    xd, wqd, e8d = x.cuda(), torch.from_numpy(wq).cuda(), torch.from_numpy(e8).cuda()
    y32 = run_blk32(xd, wqd, e8d, torch.float32)
    yh = run_blk32(xd, wqd, e8d, torch.float16)
    del xd, wqd
    assert torch.isfinite(yh).all()
    rm = _rows(M)
    for band in sorted({0, N // 32 - 1}):           # whole 32-row bands: the oracle takes N % 32 == 0
        rn = list(range(32 * band, 32 * band + 32))
        y0 = oracle.gemm_w8a16_blk32_ue8m0(f32(x[rm]), wq[rn], e8[band:band + 1])
        assert_fp32_bar(_pick(y32, rm, rn), y0, f"blk32 M={M} N={N} K={K} band {band}")
        assert_16bit_bar(_pick(yh, rm, rn), _pick(y32, rm, rn), y0, "f16", f"blk32 M={M} N={N} K={K} band {band}")
