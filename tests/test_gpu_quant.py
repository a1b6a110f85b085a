"""GPU parity of the block quantisers: codes and scales bit-exact against the
oracle on the same seeded inputs."""

import numpy as np
import pytest
import torch

import blockwise_scaled_fp8_amd as bfp8
from blockwise_scaled_fp8_amd import inputs
import oracle
from tests.gpu_helpers import say, f32

pytestmark = pytest.mark.gpu


def _act_case(x, what):
    say("quant_act", what, tuple(x.shape), x.dtype)
    xq, xs = bfp8.quantize_act(x.cuda())
    torch.cuda.synchronize()
    ref_q, ref_s = oracle.quantize_act_1x128(f32(x))
    np.testing.assert_array_equal(xs.cpu().numpy().view(np.uint32), ref_s.view(np.uint32), err_msg=what)
    np.testing.assert_array_equal(xq.cpu().numpy(), ref_q, err_msg=what)


def test_quant_act_workload0(gpu_lib):
    _act_case(inputs.workload(0)["x"], "workload 0")


@pytest.mark.parametrize("M,K", [(1, 4096), (3, 200), (5, 1000), (7, 8), (17, 136), (64, 384)])
def test_quant_act_shapes_and_ragged_groups(gpu_lib, M, K):
    _act_case(inputs.activations(M, K, workload=100 + M, stream=K), f"ragged M={M} K={K}")


def test_quant_act_fp16_input(gpu_lib):
    _act_case(inputs.activations(6, 640, workload=7, stream=0, dtype=torch.float16), "fp16")


def test_quant_act_special_groups(gpu_lib):
    x = inputs.activations(4, 512, workload=8, stream=0).float()
    x[0, :128] = 0.0                       # zero group
    x[0, 128:256] = -0.0                   # negative-zero group
    x[1, :128] *= 1e-30                    # tiny values (subnormal-range quotients stay exact)
    x[2, 5] = 0.0
    x[2, 6] = -0.0                         # signed zeros inside a live group
    x[3, :] = torch.where(torch.arange(512) % 2 == 0, x[3, :], -x[3, :])
    _act_case(x.to(torch.bfloat16), "special groups")


def test_quant_act_encoder_exhaustive_over_bf16(gpu_lib):
    """Every bf16 value in [-448, 448]: each group holds 448 (so s = 1 exactly
    and x / s = x) plus 127 values to encode."""
    b = torch.arange(0, 0x8000, dtype=torch.int32).to(torch.int16).view(torch.bfloat16)
    v = b.float()
    v = v[(v <= 448.0) & torch.isfinite(v)]
    vals = torch.cat([v, -v])
    per = 127
    rows = (vals.numel() + per - 1) // per
    pad = rows * per - vals.numel()
    vals = torch.cat([vals, torch.zeros(pad)]).reshape(rows, per)
    grid = torch.cat([torch.full((rows, 1), 448.0), vals], dim=1)     # [rows, 128]
    _act_case(grid.to(torch.bfloat16), f"exhaustive bf16 ({rows} groups)")


def test_quant_act_wide_scale_range_many_groups(gpu_lib):
    """65536 groups whose scales span about 2^-91 .. 2^102, including groups next
    to the limits of the one-division-per-group path and groups that mix
    bf16 subnormals with a normal maximum: every code and scale bit-exact."""
    M, K = 2048, 4096
    g = np.random.default_rng(77)
    z = g.standard_normal((M, K)).astype(np.float32)
    row_exp = g.integers(-60, 61, size=M).astype(np.float32)
    row_exp[:16] = np.linspace(-85, -78, 16)          # s = amax/448 on both sides of 2^-90
    row_exp[16:32] = np.linspace(104, 111, 16)       # s on both sides of 2^100
    x = z * np.exp2(row_exp)[:, None]
    x[32:48] = z[32:48] * np.float32(2.0 ** -133)    # bf16 subnormals ...
    x[32:48, ::128] = np.float32(2.0 ** -100)       # ... next to a normal group maximum
    x[48:64, :] = np.float32(0.0)                    # zero rows
    _act_case(torch.from_numpy(x).to(torch.bfloat16), "wide scale range")


def test_quant_act_prefill_outliers_sampled(gpu_lib):
    """Full 4096x4096 run with 1% outlier channels; 64 sampled rows checked."""
    x = inputs.workload(2)["x"]
    say("quant_act", "workload 2 full, sampled rows")
    xq, xs = bfp8.quantize_act(x.cuda())
    torch.cuda.synchronize()
    rows = np.random.default_rng(2).choice(4096, 64, replace=False)
    ref_q, ref_s = oracle.quantize_act_1x128(f32(x[rows]))
    np.testing.assert_array_equal(xs.cpu().numpy()[rows].view(np.uint32), ref_s.view(np.uint32))
    np.testing.assert_array_equal(xq.cpu().numpy()[rows], ref_q)


def _weight_case(w, what):
    say("quant_weight", what, tuple(w.shape), w.dtype)
    wq, ws = bfp8.quantize_weight(w.cuda())
    torch.cuda.synchronize()
    ref_q, ref_s = oracle.quantize_weight_128x128(f32(w))
    np.testing.assert_array_equal(ws.cpu().numpy().view(np.uint32), ref_s.view(np.uint32), err_msg=what)
    np.testing.assert_array_equal(wq.cpu().numpy(), ref_q, err_msg=what)


def test_quant_weight_workload0(gpu_lib):
    _weight_case(inputs.workload(0)["w"], "workload 0")


@pytest.mark.parametrize("N,K", [(200, 264), (16, 128), (384, 1000), (130, 8)])
def test_quant_weight_ragged(gpu_lib, N, K):
    _weight_case(inputs.weights_bf16(N, K, workload=200 + N, stream=K), f"ragged N={N} K={K}")


def test_quant_weight_fp16_and_zero_tile(gpu_lib):
    w = inputs.weights_bf16(256, 256, workload=9).float()
    w[:128, 128:] = 0.0
    _weight_case(w.to(torch.float16), "fp16 with a zero tile")


def test_quant_weight_full_oproj_sampled(gpu_lib):
    w = inputs.workload(1)["w"]
    say("quant_weight", "4096x4096, sampled tiles")
    wq, ws = bfp8.quantize_weight(w.cuda())
    torch.cuda.synchronize()
    for nb, kb in [(0, 0), (7, 31), (31, 0), (13, 17)]:
        blk = w[128 * nb:128 * nb + 128, 128 * kb:128 * kb + 128]
        ref_q, ref_s = oracle.quantize_weight_128x128(f32(blk))
        assert ws.cpu().numpy()[nb, kb].view(np.uint32) == ref_s[0, 0].view(np.uint32)
        np.testing.assert_array_equal(wq.cpu().numpy()[128 * nb:128 * nb + 128, 128 * kb:128 * kb + 128], ref_q)


def test_quant_deterministic(gpu_lib):
    x = inputs.activations(33, 4096, workload=10).cuda()
    a = bfp8.quantize_act(x)
    b = bfp8.quantize_act(x)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1].view(torch.int32), b[1].view(torch.int32))


# ------------------------------------------------- load-time dequantisation ----

def _dq_case(wq, scales, block, what):
    wq_d, s_d = torch.from_numpy(wq).cuda(), torch.from_numpy(scales).cuda()
    p = oracle.dequantize_weight(wq, scales, block)
    expect = {torch.float32: p, torch.bfloat16: oracle.round_bf16(p), torch.float16: oracle.round_f16(p)}
    for dt, ref in expect.items():
        say("dequant", what, block, dt)
        got = bfp8.dequantize_weight(wq_d, s_d, block, dt).float().cpu().numpy()
        ref = np.asarray(ref, np.float32)
        nan = np.isnan(ref)
        np.testing.assert_array_equal(np.isnan(got), nan, err_msg=f"{what} {dt} NaN positions")
        np.testing.assert_array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32), err_msg=f"{what} {dt}")


@pytest.mark.parametrize("block,N,K", [(32, 96, 160), (128, 200, 264), (32, 64, 8), (128, 130, 1000)])
def test_dequantize_weight_bit_exact(gpu_lib, block, N, K):
    """Every code (NaN codes included), scales of every magnitude and
    significand (powers of two in and out of the [SM70] window, values with
    full 24-bit significands), ragged edge blocks; outputs overflowing fp16
    included."""
    rng = np.random.default_rng(block * 1000 + N + K)
    wq = rng.integers(0, 256, size=(N, K), dtype=np.uint8)
    wq[0, :min(K, 256)] = np.arange(min(K, 256), dtype=np.uint8)
    nb, kb = -(-N // block), -(-K // block)
    scales = (np.exp2(rng.uniform(-40, 12, size=(nb, kb))) * rng.uniform(1, 2, size=(nb, kb))).astype(np.float32)
    scales.flat[0] = 2.0 ** -20          # a power of two below the window
    _dq_case(wq, scales, block, f"N={N} K={K}")


def test_dequantize_weight_block32_workload_shape(gpu_lib):
    """The block-32 layer shape, N = 4096, K = 7168, with scales that are not
    powers of two (the layers the packer refuses)."""
    rng = np.random.default_rng(3)
    wq = inputs.block32_codes(4096, 7168, workload=3).numpy()
    scales = (np.exp2(rng.integers(-14, 8, size=(128, 224))) * rng.uniform(1, 2, size=(128, 224))).astype(np.float32)
    _dq_case(wq, scales, 32, "block-32 layer")


def test_refused_layer_falls_back_to_blk128(gpu_lib):
    """A block-32 layer with a scale outside the window: the packer refuses it;
    dequantised to bf16 and requantised to 128x128 tiles on the GPU it matches
    the oracle's same chain bit for bit, and the W8A16 blk128 GEMM on it meets
    the bar against the oracle."""
    N, K, M = 512, 1024, 4
    wq = inputs.block32_codes(N, K, workload=31).numpy()
    s = inputs.block32_scales(N, K, workload=31).numpy()
    s[3, 5] = 2.0 ** 9                                          # outside [2^-14, 2^7]
    st, e8, bad = bfp8.bfp8_prepare_blk32_ue8m0(torch.from_numpy(wq), torch.from_numpy(s))
    assert (st, e8, bad) == (8, None, 3 * (K // 32) + 5)        # BFP8_E_SCALE_WINDOW at scale [3, 5]
    say("fallback: dequant + requant")
    w_bf16 = bfp8.dequantize_weight(torch.from_numpy(wq).cuda(), torch.from_numpy(s).cuda(), 32, torch.bfloat16)
    wq2, ws2 = bfp8.quantize_weight(w_bf16)
    ref_w = oracle.round_bf16(oracle.dequantize_weight(wq, s, 32))
    ref_q, ref_s = oracle.quantize_weight_128x128(ref_w)
    np.testing.assert_array_equal(wq2.cpu().numpy(), ref_q)
    np.testing.assert_array_equal(ws2.cpu().numpy().view(np.uint32), ref_s.view(np.uint32))
    x = inputs.activations(M, K, workload=31, dtype=torch.bfloat16)
    y = bfp8.gemm_w8a16(x.cuda(), wq2, ws2, out_dtype=torch.float32)
    y0 = oracle.gemm_w8a16_blk128(f32(x), ref_q, ref_s)
    ok, err = oracle.check_gemm_fp32(y.cpu().numpy(), y0)
    assert ok, err
