"""GPU parity of the three block-scaled GEMMs against the float64 oracle on the
same seeded inputs.

The binding bar is on the fp32-output mode (max |err| <= 1e-2 * rms(Y0) and
relative Frobenius error <= 4e-3).  16-bit outputs must meet the per-element
bar widened by half an output ulp and equal round-to-nearest-even of the
kernel's own fp32 result bit for bit.  One-hot cases are exact."""

import numpy as np
import pytest
import torch

import blockwise_scaled_fp8_amd as bfp8
from blockwise_scaled_fp8_amd import inputs
import oracle
from tests.gpu_helpers import (FINITE_CODES, say, dev, f32, workspace, run_w8a8, run_w8a16, run_blk32,
                               assert_fp32_bar, assert_16bit_bar)
from tests import cases
from tests.cases import expect, W8A8, QW8A8, W8A16, BLK32

pytestmark = pytest.mark.gpu


def _w8a8_inputs(M, N, K, wid, outliers=False):
    x = inputs.activations(M, K, workload=wid, stream=0, outliers=outliers)
    w = inputs.weights_bf16(N, K, workload=wid, stream=1)
    xq, xs = oracle.quantize_act_1x128(f32(x))
    wq, ws = oracle.quantize_weight_128x128(f32(w))
    return xq, xs, wq, ws


def _w8a8_check(M, N, K, wid, outliers=False, what="", kernel=None):
    say("w8a8", what, f"M={M} N={N} K={K}", kernel)
    if kernel is not None:
        expect(W8A8, M, N, K, kernel)
    xq, xs, wq, ws = _w8a8_inputs(M, N, K, wid, outliers)
    y0 = oracle.gemm_w8a8_blk128(xq, xs, wq, ws)
    d = [dev(a) for a in (xq, xs, wq, ws)]
    y32 = run_w8a8(*d, torch.float32)
    assert_fp32_bar(y32, y0, f"w8a8 {what} M={M} N={N} K={K}")
    y16 = run_w8a8(*d, torch.bfloat16)
    assert_16bit_bar(y16, y32, y0, "bf16", f"w8a8 {what}")
    yh = run_w8a8(*d, torch.float16)
    assert_16bit_bar(yh, y32, y0, "f16", f"w8a8 {what}")
    return y32


def test_w8a8_workload0(gpu_lib):
    _w8a8_check(4, 512, 512, 0, what="workload 0", kernel="w8a8_stream")


@pytest.mark.parametrize("M,N,K,kernel", cases.W8A8_THRESHOLD)
def test_w8a8_across_the_stream_tile_threshold(gpu_lib, M, N, K, kernel):
    _w8a8_check(M, N, K, 300 + M, what="threshold", kernel=kernel)


@pytest.mark.parametrize("M,N,K,kernel", cases.W8A8_ONE_TOKEN)
def test_w8a8_one_token(gpu_lib, M, N, K, kernel):
    """M = 1 with K <= 8192: the vector-ALU dot-product kernel (one weight
    row per wave, four or eight 1 KB chunks per lane), with K of one
    block and K ending inside a chunk; no workspace."""
    assert bfp8.bfp8_workspace_bytes(bfp8.OP_GEMM_W8A8_BLK128, 1, N, K) == 0
    _w8a8_check(1, N, K, 450 + N + K // 128, what="one token", kernel=kernel)


@pytest.mark.parametrize("M,N,K,kernel", cases.W8A8_ABOVE_ONE_TOKEN)
def test_w8a8_one_token_above_its_range(gpu_lib, M, N, K, kernel):
    """M = 1 just above K = 8192 streams (split K on the narrow projection)."""
    _w8a8_check(1, N, K, 470 + N + K // 128, what="above one token", kernel=kernel)


@pytest.mark.parametrize("M,N,K,kernel", cases.W8A8_STRADDLE)
def test_w8a8_weight_scale_rows_straddle(gpu_lib, M, N, K, kernel):
    """N not a multiple of 128: tiles straddle or subdivide a 128-row weight-scale block."""
    _w8a8_check(M, N, K, 400 + N + M, what="straddle", kernel=kernel)


@pytest.mark.parametrize("M,N,K,kernel", cases.W8A8_SPLIT_K_STREAM)
def test_w8a8_split_k_narrow_projection(gpu_lib, M, N, K, kernel):
    """N=512, K=12288 streams with K split over workgroups; run twice (counters re-arm)."""
    expect(W8A8, M, N, K, kernel)
    assert bfp8.bfp8_workspace_bytes(bfp8.OP_GEMM_W8A8_BLK128, M, 512, 12288) > 0
    xq, xs, wq, ws = _w8a8_inputs(M, 512, 12288, 500 + M)
    y0 = oracle.gemm_w8a8_blk128(xq, xs, wq, ws)
    d = [dev(a) for a in (xq, xs, wq, ws)]
    wsb = workspace(bfp8.OP_GEMM_W8A8_BLK128, M, 512, 12288)
    say("w8a8 split-K", M)
    y1 = run_w8a8(*d, torch.float32, wsb)
    y2 = run_w8a8(*d, torch.float32, wsb)
    assert_fp32_bar(y1, y0, "split-K")
    assert torch.equal(y1.view(torch.int32), y2.view(torch.int32))


@pytest.mark.parametrize("M,N,K,kernel", cases.W8A8_NO_WORKSPACE)
def test_w8a8_wide_all_tokens(gpu_lib, M, N, K, kernel):
    """The paths that need no workspace for M <= 512: the kernel that holds
    every token of a group per 16-, 32- or 64-row weight tile (one 16-token
    tile for M <= 16 where streaming would split K or take several rounds;
    groups of 32 or 64 tokens for 16 < M <= 32, and K <=
    4096 where its launch fits one round) and the streaming kernel over
    16-token tiles on small projections (grid.z, e.g. N = 1024 or 16 at
    M <= 64); ragged M inside the last token tile and in a further token
    group, a single 16-row weight tile, 64-row tiles with only 16 live rows
    (N = 8208, 2064), one K block for four waves, and K spread unevenly over
    the waves."""
    assert bfp8.bfp8_workspace_bytes(bfp8.OP_GEMM_W8A8_BLK128, M, N, K) == 0
    _w8a8_check(M, N, K, 900 + M, what="wide", kernel=kernel)


@pytest.mark.parametrize("M,N,K,kernel", cases.W8A8_WIDE_SPLIT)
def test_w8a8_wide_split_k(gpu_lib, M, N, K, kernel):
    """Long K on the all-token kernel with K split over two or four
    workgroups: the last part of each tile to arrive sums the parts in split
    order and re-arms its counter, so two calls on one workspace give the
    same bits; ragged M, an uneven split, K = 16384, one token."""
    say("w8a8 wide split", kernel, f"M={M} N={N} K={K}")
    expect(W8A8, M, N, K, kernel)
    xq, xs, wq, ws = _w8a8_inputs(M, N, K, 1300 + M)
    y0 = oracle.gemm_w8a8_blk128(xq, xs, wq, ws)
    d = [dev(a) for a in (xq, xs, wq, ws)]
    wsb = workspace(bfp8.OP_GEMM_W8A8_BLK128, M, N, K)
    assert wsb is not None
    y1 = run_w8a8(*d, torch.float32, wsb)
    assert_fp32_bar(y1, y0, f"wide split {kernel} M={M} N={N} K={K}")
    y16 = run_w8a8(*d, torch.bfloat16, wsb)
    assert_16bit_bar(y16, y1, y0, "bf16", f"wide split {kernel}")
    y2 = run_w8a8(*d, torch.float32, wsb)
    assert torch.equal(y1.view(torch.int32), y2.view(torch.int32))


@pytest.mark.parametrize("M,N,K,shape", cases.W8A8_TILE)
def test_w8a8_tile_shapes_and_split_k(gpu_lib, M, N, K, shape):
    """Every tiled configuration, with ragged M and N tiles and split K; the
    split plans run twice on one workspace (counters re-arm) and must repeat
    bit for bit."""
    say("w8a8 tile", shape, f"M={M} N={N} K={K}")
    expect(W8A8, M, N, K, shape)
    xq, xs, wq, ws = _w8a8_inputs(M, N, K, 700 + M)
    y0 = oracle.gemm_w8a8_blk128(xq, xs, wq, ws)
    d = [dev(a) for a in (xq, xs, wq, ws)]
    wsb = workspace(bfp8.OP_GEMM_W8A8_BLK128, M, N, K)
    assert (wsb is not None) == ("split" in shape)
    y1 = run_w8a8(*d, torch.float32, wsb)
    assert_fp32_bar(y1, y0, f"tile {shape}")
    y16 = run_w8a8(*d, torch.bfloat16, wsb)
    assert_16bit_bar(y16, y1, y0, "bf16", f"tile {shape}")
    y2 = run_w8a8(*d, torch.float32, wsb)
    assert torch.equal(y1.view(torch.int32), y2.view(torch.int32))


def test_w8a8_large_tile_ragged_sampled(gpu_lib):
    """256x256 tiles with ragged M and N (N straddles weight-scale rows):
    full GPU run, oracle on sampled rows including the last tile's."""
    M, N, K, kernel = cases.W8A8_LARGE_RAGGED
    say("w8a8 256x256 ragged", M, N, K)
    expect(W8A8, M, N, K, kernel)
    xq, xs, wq, ws = _w8a8_inputs(M, N, K, 800)
    y32 = run_w8a8(*(dev(a) for a in (xq, xs, wq, ws)), torch.float32)
    rows = np.concatenate([np.random.default_rng(4).choice(3840, 24, replace=False), np.arange(3840, 4000, 5)])
    y0 = oracle.gemm_w8a8_blk128(xq[rows], xs[rows], wq, ws)
    assert_fp32_bar(y32[rows], y0, "256x256 ragged sampled rows")


@pytest.mark.parametrize("xdtype", [torch.bfloat16, torch.float16])
@pytest.mark.parametrize("M,N,K,kernel", cases.QUANT_W8A8)
def test_quant_gemm_equals_quantise_then_gemm(gpu_lib, M, N, K, kernel, xdtype):
    """The fused call is bit-identical to bfp8_quantize_act_1x128 followed by
    bfp8_gemm_w8a8_blk128 (fp32 and 16-bit outputs), and meets the oracle bar.
    bf16 cases include a zero row (a zero group at M = 1) and rows (groups)
    whose scales lie outside [2^-90, 2^100] (the quantiser's IEEE-division
    path)."""
    say("quant+w8a8", xdtype, f"M={M} N={N} K={K}", kernel)
    expect(QW8A8, M, N, K, kernel)
    x = inputs.activations(M, K, workload=900 + M, stream=K, outliers=True, dtype=xdtype).float()
    if xdtype == torch.bfloat16 and M >= 3:
        x[0] = 0.0
        x[1] *= 2.0 ** -100
        x[2] *= 2.0 ** 110
    if xdtype == torch.bfloat16 and M == 1 and K >= 512:
        x[0, :128] = 0.0
        x[0, 256:384] *= 2.0 ** -100
        x[0, 384:512] *= 2.0 ** 110
    x = x.to(xdtype)
    wq, ws = oracle.quantize_weight_128x128(f32(inputs.weights_bf16(N, K, workload=900 + N, stream=K)))
    wqd, wsd, xd = dev(wq), dev(ws), x.cuda()
    xq, xs = bfp8.quantize_act(xd)
    wsb = workspace(bfp8.OP_QUANT_GEMM_W8A8_BLK128, M, N, K)
    for out in (torch.float32, torch.bfloat16):
        ref = run_w8a8(xq, xs, wqd, wsd, out)
        y = torch.empty((M, N), dtype=out, device="cuda")
        bfp8.bfp8_quant_gemm_w8a8_blk128(xd, wqd, wsd, y, wsb)
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16 if out != torch.float32 else torch.int32),
                           ref.view(torch.int16 if out != torch.float32 else torch.int32)), out
        if out == torch.float32:
            q0, s0 = oracle.quantize_act_1x128(f32(x))
            np.testing.assert_array_equal(xq.cpu().numpy(), q0)
            assert_fp32_bar(y, oracle.gemm_w8a8_blk128(q0, s0, wq, ws), f"quant+w8a8 M={M}")


def test_w8a8_decode_oproj_full(gpu_lib):
    """Decode o_proj M=1, N=K=4096: full oracle."""
    M, N, K, kernel = cases.W8A8_DECODE_OPROJ
    _w8a8_check(M, N, K, 1, what="o_proj decode", kernel=kernel)


def test_w8a8_prefill_oproj_sampled(gpu_lib):
    """Prefill o_proj M=N=K=4096 with 1% outlier channels: full GPU run, 64 rows checked."""
    say("w8a8 prefill full size")
    expect(W8A8, *cases.W8A8_PREFILL_OPROJ)
    x = inputs.workload(2)["x"]
    w = inputs.workload(2)["w"]
    xq_d, xs_d = bfp8.quantize_act(x.cuda())
    wq_d, ws_d = bfp8.quantize_weight(w.cuda())
    y32 = run_w8a8(xq_d, xs_d, wq_d, ws_d, torch.float32)
    y16 = run_w8a8(xq_d, xs_d, wq_d, ws_d, torch.bfloat16)
    rows = np.random.default_rng(3).choice(4096, 64, replace=False)
    xq, xs = oracle.quantize_act_1x128(f32(x[rows]))
    wq, ws = oracle.quantize_weight_128x128(f32(w))
    # the GPU quantisers are bit-exact (checked elsewhere); confirm on the sampled rows
    np.testing.assert_array_equal(xq_d.cpu().numpy()[rows], xq)
    np.testing.assert_array_equal(wq_d.cpu().numpy(), wq)
    y0 = oracle.gemm_w8a8_blk128(xq, xs, wq, ws)
    assert_fp32_bar(y32[rows], y0, "prefill sampled rows")
    assert_16bit_bar(y16[rows], y32[rows], y0, "bf16", "prefill sampled rows")


@pytest.mark.parametrize("M,N,K,kernel", cases.W8A8_ONE_HOT)
def test_w8a8_one_hot_all_codes_exact(gpu_lib, M, N, K, kernel):
    """xq one-hot 1.0 at column k, unit scales: Y[:, n] = E4M3(wq[n, k]) exactly,
    for every finite code (one-token and stream kernels)."""
    expect(W8A8, M, N, K, kernel)
    wq = np.zeros((N, K), np.uint8)
    wq[:254, :] = FINITE_CODES[:, None]
    for k in (0, 77, 128, 255):
        say("w8a8 one-hot", M, k)
        xq = np.zeros((M, K), np.uint8)
        xq[:, k] = 0x38
        y = run_w8a8(dev(xq), dev(np.ones((M, 2), np.float32)), dev(wq), dev(np.ones((2, 2), np.float32)),
                     torch.float32)
        want = np.broadcast_to(oracle.e4m3_decode(wq[:, k]), (M, N))
        np.testing.assert_array_equal(y.cpu().numpy(), want)


def test_w8a8_deterministic(gpu_lib):
    M, N, K, kernel = cases.W8A8_DETERMINISTIC
    expect(W8A8, M, N, K, kernel)
    xq, xs, wq, ws = _w8a8_inputs(M, N, K, 11)
    d = [dev(a) for a in (xq, xs, wq, ws)]
    a = run_w8a8(*d, torch.float32)
    b = run_w8a8(*d, torch.float32)
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))


# ------------------------------------------------------------ W8A16 blk128 ----

@pytest.mark.parametrize("xdtype", [torch.bfloat16, torch.float16])
@pytest.mark.parametrize("M,N,K,kernel", cases.W8A16_BY_M)
def test_w8a16_blk128(gpu_lib, M, N, K, kernel, xdtype):
    say("w8a16 blk128", M, xdtype, kernel)
    expect(W8A16, M, N, K, kernel)
    x = inputs.activations(M, K, workload=600 + M, dtype=xdtype)
    wq, ws = oracle.quantize_weight_128x128(f32(inputs.weights_bf16(N, K, workload=600 + M)))
    y0 = oracle.gemm_w8a16_blk128(f32(x), wq, ws)
    xd, wqd, wsd = x.cuda(), dev(wq), dev(ws)
    y32 = run_w8a16(xd, wqd, wsd, torch.float32)
    assert_fp32_bar(y32, y0, f"w8a16 M={M}")
    y16 = run_w8a16(xd, wqd, wsd, xdtype)
    assert_16bit_bar(y16, y32, y0, "bf16" if xdtype == torch.bfloat16 else "f16", f"w8a16 M={M}")


@pytest.mark.parametrize("xdtype", [torch.bfloat16, torch.float16])
@pytest.mark.parametrize("M,N,K,kernel", cases.W8A16_ONE_TOKEN)
def test_w8a16_gemv_one_token(gpu_lib, M, N, K, kernel, xdtype):
    """M = 1 with K <= 12288: the vector-ALU dot-product kernel, one weight
    row per wave, 4, 8 or 12 chunks of 1 KB per lane; a K of one
    block, K ending inside a chunk (1152, 3968, 5120), N of one workgroup;
    all three output types."""
    say("w8a16 gemv", xdtype, f"N={N} K={K}")
    expect(W8A16, M, N, K, kernel)
    assert bfp8.bfp8_workspace_bytes(bfp8.OP_GEMM_W8A16_BLK128, 1, N, K) == 0
    x = inputs.activations(1, K, workload=660 + N, stream=K, outliers=True, dtype=xdtype)
    wq, ws = oracle.quantize_weight_128x128(f32(inputs.weights_bf16(N, K, workload=661, stream=K)))
    y0 = oracle.gemm_w8a16_blk128(f32(x), wq, ws)
    xd, wqd, wsd = x.cuda(), dev(wq), dev(ws)
    y32 = run_w8a16(xd, wqd, wsd, torch.float32)
    assert_fp32_bar(y32, y0, f"w8a16 gemv N={N} K={K}")
    for out in (torch.bfloat16, torch.float16):
        y16 = run_w8a16(xd, wqd, wsd, out)
        assert_16bit_bar(y16, y32, y0, "bf16" if out == torch.bfloat16 else "f16", f"w8a16 gemv N={N} K={K}")


@pytest.mark.parametrize("xdtype", [torch.bfloat16, torch.float16])
@pytest.mark.parametrize("M,N,K,kernel", cases.W8A16_ONE_TILE)
def test_w8a16_one_token_tile(gpu_lib, M, N, K, kernel, xdtype):
    """8 < M <= 16 without a split of K, and 4 <= M <= 8 where streaming
    would take several rounds: the all-token kernel with a single 16-token
    tile (token rows of a ragged M past the end load as zeros), one, two or
    four weight-row tiles per workgroup (a last tile with 16 live rows), K of
    one block and long K; no workspace."""
    assert bfp8.bfp8_workspace_bytes(bfp8.OP_GEMM_W8A16_BLK128, M, N, K) == 0
    say("w8a16 one tile", xdtype, f"M={M} N={N} K={K}")
    expect(W8A16, M, N, K, kernel)
    x = inputs.activations(M, K, workload=670 + M, stream=K, outliers=True, dtype=xdtype)
    wq, ws = oracle.quantize_weight_128x128(f32(inputs.weights_bf16(N, K, workload=670 + N, stream=K)))
    y0 = oracle.gemm_w8a16_blk128(f32(x), wq, ws)
    xd, wqd, wsd = x.cuda(), dev(wq), dev(ws)
    y32 = run_w8a16(xd, wqd, wsd, torch.float32)
    assert_fp32_bar(y32, y0, f"w8a16 one tile M={M} N={N} K={K}")
    y16 = run_w8a16(xd, wqd, wsd, xdtype)
    assert_16bit_bar(y16, y32, y0, "bf16" if xdtype == torch.bfloat16 else "f16", f"w8a16 one tile M={M}")
    y2 = run_w8a16(xd, wqd, wsd, torch.float32)
    assert torch.equal(y32.view(torch.int32), y2.view(torch.int32))


@pytest.mark.parametrize("xdtype", [torch.bfloat16, torch.float16])
@pytest.mark.parametrize("M,N,K,kernel", cases.W8A16_ALL_TOKENS)
def test_w8a16_all_tokens(gpu_lib, M, N, K, kernel, xdtype):
    """16 < M <= 256 with K <= 4096: every token of a group per 16- or 32-row
    weight tile, no workspace.  Covers one and two weight-row tiles per
    workgroup (a half-filled last pair at N = 16 and 4112), two and four
    token tiles, several token groups (grid.y) with a ragged last group and
    an empty last tile (M = 100), and K spread over the waves."""
    assert bfp8.bfp8_workspace_bytes(bfp8.OP_GEMM_W8A16_BLK128, M, N, K) == 0
    say("w8a16 all-token", xdtype, f"M={M} N={N} K={K}")
    expect(W8A16, M, N, K, kernel)
    x = inputs.activations(M, K, workload=640 + M, stream=K, outliers=True, dtype=xdtype)
    wq, ws = oracle.quantize_weight_128x128(f32(inputs.weights_bf16(N, K, workload=640 + N, stream=K)))
    y0 = oracle.gemm_w8a16_blk128(f32(x), wq, ws)
    xd, wqd, wsd = x.cuda(), dev(wq), dev(ws)
    y32 = run_w8a16(xd, wqd, wsd, torch.float32)
    assert_fp32_bar(y32, y0, f"w8a16 all-token M={M}")
    y16 = run_w8a16(xd, wqd, wsd, xdtype)
    assert_16bit_bar(y16, y32, y0, "bf16" if xdtype == torch.bfloat16 else "f16", f"w8a16 all-token M={M}")


@pytest.mark.parametrize("M,N,K,kernel", cases.W8A16_LONG_K + cases.W8A16_SPLIT_K_STREAM)
def test_w8a16_blk128_long_k(gpu_lib, M, N, K, kernel):
    """K = 12288: six 128-K blocks per wave on 4096 rows (two passes of up to
    four blocks, the cross-wave sum in the slab memory), and K split over
    workgroups on 512 rows, run twice on one workspace (counters re-arm,
    bit-identical)."""
    say("w8a16 long K", M, N, kernel)
    expect(W8A16, M, N, K, kernel)
    x = inputs.activations(M, K, workload=650 + M, dtype=torch.bfloat16)
    wq, ws = oracle.quantize_weight_128x128(f32(inputs.weights_bf16(N, K, workload=651)))
    y0 = oracle.gemm_w8a16_blk128(f32(x), wq, ws)
    wsb = workspace(bfp8.OP_GEMM_W8A16_BLK128, M, N, K)
    assert (wsb is not None) == kernel.endswith("/split")
    y32 = run_w8a16(x.cuda(), dev(wq), dev(ws), torch.float32, wsb)
    assert_fp32_bar(y32, y0, f"w8a16 long K M={M}")
    y2 = run_w8a16(x.cuda(), dev(wq), dev(ws), torch.float32, wsb)
    assert torch.equal(y32.view(torch.int32), y2.view(torch.int32))


@pytest.mark.parametrize("xdtype", [torch.bfloat16, torch.float16])
@pytest.mark.parametrize("M,N,K,kernel", cases.W8A16_ONE_HOT)
def test_w8a16_blk128_one_hot_all_codes_exact(gpu_lib, xdtype, M, N, K, kernel):
    """x one-hot 1.0: Y[:, n] = E4M3(wq[n, k]) * ws exactly, subnormal codes
    included (vector-ALU kernel at M = 1, streaming kernel at M = 4,
    all-token kernel with one token tile at M = 16 and with two at M = 40)."""
    expect(W8A16, M, N, K, kernel)
    wq = np.zeros((N, K), np.uint8)
    wq[:254, :] = FINITE_CODES[:, None]
    ws = np.array([[0.5, 2.0], [0.25, 4.0]], np.float32)
    for k in (0, 100, 129, 255):
        say("w8a16 one-hot", xdtype, M, k)
        x = torch.zeros((M, K), dtype=xdtype)
        x[:, k] = 1.0
        y = run_w8a16(x.cuda(), dev(wq), dev(ws), torch.float32)
        want = oracle.e4m3_decode(wq[:, k]) * ws[np.arange(N) // 128, k // 128]
        np.testing.assert_array_equal(y.cpu().numpy(), np.broadcast_to(want, (M, N)))


@pytest.mark.parametrize("xdtype", [torch.bfloat16, torch.float16])
@pytest.mark.parametrize("M,N,K,kernel", cases.W8A16_TILE_SPLIT)
def test_w8a16_tile_split_k(gpu_lib, M, N, K, kernel, xdtype):
    """Tiled W8A16 with ragged M/N tiles and split K (workspace), run twice on
    one workspace: bar met, second run bit-identical (and one 128 x 64 plan
    with enough tiles that K is not split)."""
    say("w8a16 tile", xdtype, f"M={M} N={N} K={K}", kernel)
    expect(W8A16, M, N, K, kernel)
    x = inputs.activations(M, K, workload=620 + M, stream=K, outliers=True, dtype=xdtype)
    wq, ws = oracle.quantize_weight_128x128(f32(inputs.weights_bf16(N, K, workload=620 + N, stream=K)))
    y0 = oracle.gemm_w8a16_blk128(f32(x), wq, ws)
    xd, wqd, wsd = x.cuda(), dev(wq), dev(ws)
    wsb = workspace(bfp8.OP_GEMM_W8A16_BLK128, M, N, K)
    y1 = run_w8a16(xd, wqd, wsd, torch.float32, wsb)
    assert_fp32_bar(y1, y0, f"w8a16 tile M={M}")
    y2 = run_w8a16(xd, wqd, wsd, torch.float32, wsb)
    assert torch.equal(y1.view(torch.int32), y2.view(torch.int32))
    y16 = run_w8a16(xd, wqd, wsd, xdtype, wsb)
    assert_16bit_bar(y16, y1, y0, "bf16" if xdtype == torch.bfloat16 else "f16", f"w8a16 tile M={M}")


@pytest.mark.parametrize("xdtype", [torch.bfloat16, torch.float16])
def test_w8a16_tile_one_hot_all_codes_exact(gpu_lib, xdtype):
    """Tiled path (M = 8200: no one-round all-token shape at N = 256): x
    one-hot 1.0 gives E4M3(wq[n, k]) * ws exactly."""
    M, N, K, kernel = cases.W8A16_TILE_ONE_HOT
    expect(W8A16, M, N, K, kernel)
    wq = np.zeros((N, K), np.uint8)
    wq[:254, :] = FINITE_CODES[:, None]
    ws = np.array([[0.5, 2.0], [0.25, 4.0]], np.float32)
    for k in (0, 37, 130, 255):
        say("w8a16 tile one-hot", xdtype, k)
        x = torch.zeros((M, K), dtype=xdtype)
        x[:, k] = 1.0
        y = run_w8a16(x.cuda(), dev(wq), dev(ws), torch.float32)
        want = oracle.e4m3_decode(wq[:, k]) * ws[np.arange(N) // 128, k // 128]
        np.testing.assert_array_equal(y.cpu().numpy(), np.broadcast_to(want, (M, N)))


@pytest.mark.parametrize("xdtype", [torch.bfloat16, torch.float16])
def test_w8a16_tile_large_ragged(gpu_lib, xdtype):
    """The 256 x 128 W8A16 tile (chosen once it gives 256 tiles) with a ragged
    last weight tile (N = 4112) and a ragged last token tile (M = 2000)."""
    M, N, K, kernel = cases.W8A16_TILE_LARGE_RAGGED
    say("w8a16 tile large", xdtype)
    expect(W8A16, M, N, K, kernel)
    x = inputs.activations(M, K, workload=640, stream=1, outliers=True, dtype=xdtype)
    wq, ws = oracle.quantize_weight_128x128(f32(inputs.weights_bf16(N, K, workload=641)))
    y0 = oracle.gemm_w8a16_blk128(f32(x), wq, ws)
    xd, wqd, wsd = x.cuda(), dev(wq), dev(ws)
    y32 = run_w8a16(xd, wqd, wsd, torch.float32)
    assert_fp32_bar(y32, y0, "w8a16 tile large")
    y16 = run_w8a16(xd, wqd, wsd, xdtype)
    assert_16bit_bar(y16, y32, y0, "bf16" if xdtype == torch.bfloat16 else "f16", "w8a16 tile large")


@pytest.mark.parametrize("xdtype", [torch.bfloat16, torch.float16])
def test_w8a16_tile_large_one_hot_all_codes_exact(gpu_lib, xdtype):
    """256 x 128 tile path (M = 2048, N = 4096): x one-hot 1.0 gives
    E4M3(wq[n, k]) * ws exactly, every finite code in every weight tile."""
    M, N, K, kernel = cases.W8A16_TILE_LARGE_ONE_HOT
    expect(W8A16, M, N, K, kernel)
    wq = FINITE_CODES[np.arange(N) % 254][:, None].repeat(K, axis=1).astype(np.uint8)
    ws = np.where((np.arange(N // 128)[:, None] + np.arange(K // 128)[None, :]) % 2 == 0, 0.5, 4.0).astype(np.float32)
    for k in (3, 200):
        say("w8a16 tile large one-hot", xdtype, k)
        x = torch.zeros((M, K), dtype=xdtype)
        x[:, k] = 1.0
        y = run_w8a16(x.cuda(), dev(wq), dev(ws), torch.float32)
        want = oracle.e4m3_decode(wq[:, k]) * ws[np.arange(N) // 128, k // 128]
        np.testing.assert_array_equal(y.cpu().numpy(), np.broadcast_to(want, (M, N)))


@pytest.mark.parametrize("xdtype", [torch.bfloat16, torch.float16])
def test_w8a16_prefill_oproj_sampled(gpu_lib, xdtype):
    """M = N = K = 4096 W8A16 with 1% outlier channels: full GPU run, 48 rows checked."""
    say("w8a16 prefill", xdtype)
    expect(W8A16, *cases.W8A16_PREFILL_OPROJ)
    x = inputs.activations(4096, 4096, workload=2, stream=0, outliers=True, dtype=xdtype)
    w = inputs.workload(2)["w"]
    wq_d, ws_d = bfp8.quantize_weight(w.cuda())
    y32 = run_w8a16(x.cuda(), wq_d, ws_d, torch.float32)
    rows = np.concatenate([np.random.default_rng(5).choice(4096, 40, replace=False), np.arange(4088, 4096)])
    wq, ws = oracle.quantize_weight_128x128(f32(w))
    y0 = oracle.gemm_w8a16_blk128(f32(x[rows]), wq, ws)
    assert_fp32_bar(y32[rows], y0, "w8a16 prefill sampled rows")


def test_w8a16_blk128_decode_oproj_full(gpu_lib):
    say("w8a16 o_proj decode")
    expect(W8A16, *cases.W8A16_DECODE_OPROJ)
    x = inputs.workload(1)["x"]
    wq, ws = oracle.quantize_weight_128x128(f32(inputs.workload(1)["w"]))
    y0 = oracle.gemm_w8a16_blk128(f32(x), wq, ws)
    y32 = run_w8a16(x.cuda(), dev(wq), dev(ws), torch.float32)
    assert_fp32_bar(y32, y0, "w8a16 o_proj")
    y16 = run_w8a16(x.cuda(), dev(wq), dev(ws), torch.bfloat16)
    assert_16bit_bar(y16, y32, y0, "bf16", "w8a16 o_proj")


# ------------------------------------------------------------ blk32 UE8M0 ----

def _blk32_inputs(M, N, K, wid, lo=-14, hi=7):
    x = inputs.activations(M, K, workload=wid, stream=0, dtype=torch.float16)
    wq = inputs.block32_codes(N, K, workload=wid).numpy()
    s = inputs.block32_scales(N, K, workload=wid, lo=lo, hi=hi).numpy()
    st, e8, bad = bfp8.bfp8_prepare_blk32_ue8m0(torch.from_numpy(wq), torch.from_numpy(s))
    assert st == 0, (st, bad)
    ref_st, ref_e8, _ = oracle.prepare_blk32_ue8m0(wq, s)
    np.testing.assert_array_equal(e8.numpy(), ref_e8)
    return x, wq, e8.numpy()


@pytest.mark.parametrize("M,N,K,kernel", cases.BLK32_WORKLOAD)
def test_blk32_block32_workload_shape(gpu_lib, M, N, K, kernel):
    """N=4096, K=7168 block-32 weights, e uniform on [-14, 7] (M = 1 on the
    one-token kernel, M = 2 .. 8 streaming, M = 9 .. 16 on the all-token
    kernel with one token tile)."""
    say("blk32", M)
    expect(BLK32, M, N, K, kernel)
    x, wq, e8 = _blk32_inputs(M, N, K, 3)
    y0 = oracle.gemm_w8a16_blk32_ue8m0(f32(x), wq, e8)
    xd, wqd, e8d = x.cuda(), dev(wq), dev(e8)
    y32 = run_blk32(xd, wqd, e8d, torch.float32)
    assert_fp32_bar(y32, y0, f"blk32 M={M}")
    yh = run_blk32(xd, wqd, e8d, torch.float16)
    assert_16bit_bar(yh, y32, y0, "f16", f"blk32 M={M}")
    ok, e = oracle.check_gemm_fp32(f32(yh), y0)     # fp16 half-ulp is far below the bar here
    assert ok, e


@pytest.mark.parametrize("M,N,K,kernel", cases.BLK32_ONE_TOKEN)
def test_blk32_one_token(gpu_lib, M, N, K, kernel):
    """One token with K <= 8192: the vector-ALU kernel (one row per wave, 4
    or 8 chunks), e uniform on [-14, 7], and the streaming kernel just above;
    fp32 output against the oracle, fp16 output as RNE of the fp32
    result."""
    say("blk32 one token", N, K)
    expect(BLK32, M, N, K, kernel)
    x, wq, e8 = _blk32_inputs(M, N, K, 60 + K // 128)
    y0 = oracle.gemm_w8a16_blk32_ue8m0(f32(x), wq, e8)
    xd, wqd, e8d = x.cuda(), dev(wq), dev(e8)
    y32 = run_blk32(xd, wqd, e8d, torch.float32)
    assert_fp32_bar(y32, y0, f"blk32 one token N={N} K={K}")
    yh = run_blk32(xd, wqd, e8d, torch.float16)
    assert_16bit_bar(yh, y32, y0, "f16", f"blk32 one token N={N} K={K}")


@pytest.mark.parametrize("lo,hi", [(-14, -14), (7, 7)])
def test_blk32_window_ends(gpu_lib, lo, hi):
    say("blk32 window end", lo)
    M, N, K, kernel = cases.BLK32_WINDOW
    expect(BLK32, M, N, K, kernel)
    x, wq, e8 = _blk32_inputs(M, N, K, 30 + lo, lo=lo, hi=hi)
    y0 = oracle.gemm_w8a16_blk32_ue8m0(f32(x), wq, e8)
    y32 = run_blk32(x.cuda(), dev(wq), dev(e8), torch.float32)
    assert_fp32_bar(y32, y0, f"blk32 e={lo}")


@pytest.mark.parametrize("case", [cases.BLK32_ONE_HOT, cases.BLK32_ONE_HOT_STREAM, cases.BLK32_ONE_HOT_ABOVE_16,
                                  cases.BLK32_ONE_HOT_ABOVE_16_SPLIT, cases.BLK32_TILE_ONE_HOT,
                                  cases.BLK32_ONE_HOT_ONE_TOKEN], ids=lambda c: c[3])
@pytest.mark.parametrize("out", [torch.float32, torch.float16])
def test_blk32_one_hot_all_codes_all_exponents_exact(gpu_lib, out, case):
    """Every finite code times every window exponent is produced exactly
    (fp16 subnormals at e = -14 included), by the all-token kernel with one
    token tile (M = 16) and with a group of two (M = 17: a full tile and one
    with a single live row), the streaming kernel of M <= 8, the one for
    M > 16 with K split (M = 17, K = 8320), the tiled kernel (M = 300: the
    last 128-row weight tile ends at N = 704, its waves past N reading the
    last scale band) and the one-token kernel (M = 1: one column k per
    call)."""
    exps = np.arange(-14, 8)
    M, N, K, kernel = case
    assert N == 32 * exps.size
    expect(BLK32, M, N, K, kernel)
    wq = np.zeros((N, K), np.uint8)
    wq[:, :254] = FINITE_CODES[None, :]
    e8 = np.repeat((exps + 127).astype(np.uint8)[:, None], K // 32, axis=1)
    d = oracle.e4m3_decode(FINITE_CODES)
    for base in range(0, 256, M):
        say("blk32 one-hot", out, M, base)
        x = torch.zeros((M, K), dtype=torch.float16)
        ks = np.arange(base, base + M) % K
        x[np.arange(M), ks] = 1.0
        y = run_blk32(x.cuda(), dev(wq), dev(e8), out).float().cpu().numpy()
        for row, k in enumerate(ks):
            want = (d[k] if k < 254 else 0.0) * np.exp2(exps.astype(np.float64))
            np.testing.assert_array_equal(y[row].reshape(exps.size, 32), np.repeat(want[:, None], 32, axis=1))


@pytest.mark.parametrize("case", [cases.BLK32_SPLIT_K, cases.BLK32_SPLIT_K_16, cases.BLK32_SPLIT_K_ABOVE_16],
                         ids=lambda c: f"M{c[0]}-{c[3]}")
def test_blk32_split_k_and_determinism(gpu_lib, case):
    M, N, K, kernel = case
    expect(BLK32, M, N, K, kernel)
    assert bfp8.bfp8_workspace_bytes(bfp8.OP_GEMM_W8A16_BLK32_UE8M0, M, N, K) > 0
    x, wq, e8 = _blk32_inputs(M, N, K, 31)
    y0 = oracle.gemm_w8a16_blk32_ue8m0(f32(x), wq, e8)
    wsb = workspace(bfp8.OP_GEMM_W8A16_BLK32_UE8M0, M, N, K)
    say("blk32 split-K")
    a = run_blk32(x.cuda(), dev(wq), dev(e8), torch.float32, wsb)
    b = run_blk32(x.cuda(), dev(wq), dev(e8), torch.float32, wsb)
    assert_fp32_bar(a, y0, "blk32 split-K")
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))


@pytest.mark.parametrize("M,N,K,kernel", cases.BLK32_ONE_TILE)
def test_blk32_one_token_tile(gpu_lib, M, N, K, kernel):
    """8 < M <= 16 without a split of K: the all-token kernel with one
    16-token tile, the UE8M0 scale word of each block applied in the
    widening; one and two weight-row tiles (two 16-row halves of one
    32-row scale band), ragged M, tiny N; fp32 output against the oracle,
    fp16 as RNE of the fp32 result, a rerun bit-identical."""
    say("blk32 one tile", M, N, K)
    expect(BLK32, M, N, K, kernel)
    assert bfp8.bfp8_workspace_bytes(bfp8.OP_GEMM_W8A16_BLK32_UE8M0, M, N, K) == 0
    x, wq, e8 = _blk32_inputs(M, N, K, 70 + M)
    y0 = oracle.gemm_w8a16_blk32_ue8m0(f32(x), wq, e8)
    xd, wqd, e8d = x.cuda(), dev(wq), dev(e8)
    y32 = run_blk32(xd, wqd, e8d, torch.float32)
    assert_fp32_bar(y32, y0, f"blk32 one tile M={M} N={N} K={K}")
    yh = run_blk32(xd, wqd, e8d, torch.float16)
    assert_16bit_bar(yh, y32, y0, "f16", f"blk32 one tile M={M}")
    y2 = run_blk32(xd, wqd, e8d, torch.float32)
    assert torch.equal(y32.view(torch.int32), y2.view(torch.int32))


@pytest.mark.parametrize("M,N,K,kernel", cases.BLK32_TILE)
def test_blk32_tiled(gpu_lib, M, N, K, kernel):
    """Block-32 on the W8A16 tiled kernel: 128x64, 128x128 and 256x128
    tiles, K split and not, ragged M and N; fp32 output against the oracle
    on all rows up to M = 64 and sampled rows above (the last token tile's
    rows always included), fp16 output as RNE of the fp32 result, and a
    rerun on the same workspace bit-identical."""
    say("blk32 tiled", M, N, K, kernel)
    expect(BLK32, M, N, K, kernel)
    x, wq, e8 = _blk32_inputs(M, N, K, 80 + M)
    xd, wqd, e8d = x.cuda(), dev(wq), dev(e8)
    wsb = workspace(BLK32, M, N, K)
    assert (wsb is not None) == kernel.endswith("/split")
    y32 = run_blk32(xd, wqd, e8d, torch.float32, wsb)
    yh = run_blk32(xd, wqd, e8d, torch.float16, wsb)
    y2 = run_blk32(xd, wqd, e8d, torch.float32, wsb)
    assert torch.equal(y32.view(torch.int32), y2.view(torch.int32))
    if M <= 64:
        rows = np.arange(M)
    else:
        rows = np.unique(np.concatenate([np.random.default_rng(M).choice(M, 40, replace=False),
                                         np.arange(M - 16, M)]))
    y0 = oracle.gemm_w8a16_blk32_ue8m0(f32(x[rows]), wq, e8)
    assert_fp32_bar(y32[rows], y0, f"blk32 tiled M={M} N={N} K={K}")
    assert_16bit_bar(yh[rows], y32[rows], y0, "f16", f"blk32 tiled M={M}")


@pytest.mark.parametrize("M,N,K,kernel", cases.BLK32_ABOVE_16)
def test_blk32_above_the_streaming_range(gpu_lib, M, N, K, kernel):
    """16 < M where block-32 reads all tokens of a group of 32 or 64 per 16-
    or 32-row weight tile: the workload shape (N = 4096, K = 7168) at
    M = 17 and 32, one and two row tiles, several token groups (grid.y) at
    M = 64, 100, 128 and 200, a ragged last group at M = 17, 100 and 200;
    fp32 output against the oracle (all rows up to M = 64, sampled rows
    above, the last tile's rows always included) and fp16 output as RNE of
    the fp32 result."""
    say("blk32 M > 16", M)
    expect(BLK32, M, N, K, kernel)
    x, wq, e8 = _blk32_inputs(M, N, K, 40 + M)
    xd, wqd, e8d = x.cuda(), dev(wq), dev(e8)
    y32 = run_blk32(xd, wqd, e8d, torch.float32)
    yh = run_blk32(xd, wqd, e8d, torch.float16)
    if M <= 64:
        rows = np.arange(M)
    else:
        rows = np.unique(np.concatenate([np.random.default_rng(M).choice(M, 40, replace=False),
                                         np.arange(M - 16, M)]))
    y0 = oracle.gemm_w8a16_blk32_ue8m0(f32(x[rows]), wq, e8)
    assert_fp32_bar(y32[rows], y0, f"blk32 M={M}")
    assert_16bit_bar(yh[rows], y32[rows], y0, "f16", f"blk32 M={M}")
