"""Pins for the oracle's load-time blockwise dequantisation.

Fixed by the definition w = RN_out(fl32(E4M3(q) * s)): the block map (which
scale multiplies which weight) is checked on unit codes against the scale
array expanded block by block, the per-code values against the closed-form
decode, the single fp32 rounding against exact rational products, and the bf16
/ fp16 roundings against ties constructed by hand and against torch's
conversions.  Two consequences tie it to the rest of the oracle: dequantising
the 128x128 quantiser's output returns the weights within half an E4M3 step,
and with in-window power-of-two scales ([SM70] "Exactness") the block-32 GEMM
equals a plain product with the dequantised weights, exactly.
"""

from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import (dequantize_weight, e4m3_decode, gemm_w8a16_blk32_ue8m0, prepare_blk32_ue8m0,
                    quantize_weight_128x128, round_bf16, round_f16)
from tests.test_oracle_quant import _is_round_nearest_even_f32

FINITE = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)


@pytest.mark.parametrize("block,N,K", [(32, 96, 160), (128, 200, 264), (128, 128, 128), (32, 33, 40)])
def test_block_map(block, N, K):
    rng = np.random.default_rng(block + N + K)
    nb, kb = -(-N // block), -(-K // block)
    scales = np.exp2(rng.integers(-20, 20, size=(nb, kb))).astype(np.float32)
    wq = np.full((N, K), 0x38, np.uint8)                       # every code 1.0
    expect = np.kron(scales, np.ones((block, block), np.float32))[:N, :K]
    np.testing.assert_array_equal(dequantize_weight(wq, scales, block), expect)


def test_every_code_unit_scale():
    wq = np.tile(np.arange(256, dtype=np.uint8), (32, 1))[:, :256]
    out = dequantize_weight(wq, np.ones((1, 8), np.float32), 32)
    dec = e4m3_decode(wq)
    finite = ~np.isnan(dec)
    np.testing.assert_array_equal(out[finite], dec[finite].astype(np.float32))
    assert np.isnan(out[~finite]).all() and (~finite).sum() == 2 * 32


def test_single_fp32_rounding():
    rng = np.random.default_rng(7)
    wq = FINITE[rng.integers(0, FINITE.size, size=(64, 256))]
    scales = (rng.random((2, 8)) * 3 + 0.01).astype(np.float32)   # full 24-bit significands
    out = dequantize_weight(wq, scales, 32)
    dec = e4m3_decode(wq)
    rounded = 0
    for n in range(64):
        for k in range(0, 256, 7):
            exact = Fraction(float(dec[n, k])) * Fraction(float(scales[n // 32, k // 32]))
            assert _is_round_nearest_even_f32(out[n, k], exact), (n, k)
            rounded += Fraction(float(out[n, k])) != exact
    assert rounded > 100                                            # the case is not trivially exact


def test_round_bf16_ties_and_torch():
    # 1 + 2^-8 is halfway between 1 and 1 + 2^-7 (ties to the even 1.0);
    # 1 + 3 * 2^-8 lies halfway between 1 + 2^-7 and 1 + 2^-6 (to the even 1 + 2^-6);
    # 3 * 2^-134 lies halfway between the bf16 subnormals 2^-133 and 2^-132 (to the even 2^-132).
    ties = np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, -(1 + 2.0 ** -8), 3 * 2.0 ** -134], np.float32)
    np.testing.assert_array_equal(round_bf16(ties), np.array([1.0, 1 + 2.0 ** -6, -1.0, 2.0 ** -132], np.float32))
    x = (np.random.default_rng(3).standard_normal(100000) * 50).astype(np.float32)
    np.testing.assert_array_equal(round_bf16(x), torch.from_numpy(x).to(torch.bfloat16).float().numpy())
    np.testing.assert_array_equal(round_f16(x).astype(np.float32),
                                  torch.from_numpy(x).to(torch.float16).float().numpy())


def test_round_trip_of_the_weight_quantiser():
    rng = np.random.default_rng(11)
    w = torch.from_numpy((rng.standard_normal((256, 384)) * 0.02).astype(np.float32)).to(torch.bfloat16).float().numpy()
    wq, ws = quantize_weight_128x128(w)
    dq = dequantize_weight(wq, ws, 128).astype(np.float64)
    s = np.kron(ws, np.ones((128, 128)))[:256, :384]
    # half an E4M3 step at |w|/s (2^-4 relative for normals, 2^-10 absolute
    # below 2^-6), times s, plus the fp32 roundings of the quotient and product
    bound = np.maximum(np.abs(w) * 2.0 ** -4, s * 2.0 ** -10) * (1 + 2.0 ** -20) + np.abs(w) * 2.0 ** -22
    assert (np.abs(dq - w) <= bound).all()


def test_blk32_gemm_equals_plain_product_on_dequantised_weights():
    rng = np.random.default_rng(5)
    N, K, M = 64, 128, 3
    wq = FINITE[rng.integers(0, FINITE.size, size=(N, K))]
    e = rng.integers(-14, 8, size=(N // 32, K // 32))
    scales = np.exp2(e).astype(np.float32)
    status, e8, _ = prepare_blk32_ue8m0(wq, scales)
    assert e8 is not None
    x = rng.integers(-3, 4, size=(M, K)).astype(np.float64)          # small integers: every sum exact
    y = gemm_w8a16_blk32_ue8m0(x, wq, e8)
    w = dequantize_weight(wq, scales, 32).astype(np.float64)
    assert (round_f16(w).astype(np.float64) == w).all()              # exact in fp16 inside the window
    np.testing.assert_array_equal(y, x @ w.T)
