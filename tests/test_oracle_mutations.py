"""The pins have teeth: plausible mistakes planted in copies of the oracle's
functions (on the CPU, never in the product) make at least one pin fail."""

import numpy as np
import pytest

import oracle.e4m3 as e4m3_mod
from oracle import e4m3_decode
from oracle.gemm import BLK128
import tests.test_oracle_e4m3 as pins_e4m3
import tests.test_oracle_gemm as pins_gemm


def _decode_bias8(codes):
    c = np.asarray(codes, np.uint8).astype(np.int64)
    E, m, s = (c >> 3) & 15, c & 7, c >> 7
    mag = np.where(E == 0, m * 2.0 ** -9, (1 + m / 8) * np.exp2((E - 8).astype(float)))
    return np.where((c & 0x7F) == 0x7F, np.nan, np.where(s == 1, -mag, mag))


def _decode_subnormal_as_normal(codes):
    c = np.asarray(codes, np.uint8).astype(np.int64)
    E, m, s = (c >> 3) & 15, c & 7, c >> 7
    mag = np.where(E == 0, (1 + m / 8) * 2.0 ** -6, (1 + m / 8) * np.exp2((E - 7).astype(float)))
    mag = np.where(c & 0x7F == 0, 0.0, mag)
    return np.where((c & 0x7F) == 0x7F, np.nan, np.where(s == 1, -mag, mag))


@pytest.mark.parametrize("bad", [_decode_bias8, _decode_subnormal_as_normal])
def test_decode_mistakes_are_caught(monkeypatch, bad):
    monkeypatch.setattr(pins_e4m3, "e4m3_decode", bad)
    failures = 0
    for pin in (pins_e4m3.test_decode_matches_fp16_integer_identity,
                pins_e4m3.test_decode_matches_torch_float8_e4m3fn,
                pins_e4m3.test_decode_format_facts):
        try:
            pin()
        except AssertionError:
            failures += 1
    assert failures >= 1


def _encode_ties_away(a):
    a = np.asarray(a, np.float32).astype(np.float64)
    out = e4m3_mod.e4m3_encode(a)
    # redo the rounding with ties away from zero: bump codes that were exact ties rounded down
    d = np.abs(e4m3_decode(out & 0x7F))
    up = np.abs(e4m3_decode(np.minimum((out & 0x7F) + 1, 0x7E)))
    tie_down = (np.abs(a) - d) == (up - np.abs(a))
    return np.where(tie_down & (np.abs(a) < 448), (out + 1).astype(np.uint8), out)


def _encode_no_saturation(a):
    out = e4m3_mod.e4m3_encode(a)
    big = np.abs(np.asarray(a, np.float32)) >= 464.0
    return np.where(big, out | 0x7F, out).astype(np.uint8)


@pytest.mark.parametrize("bad", [_encode_ties_away, _encode_no_saturation])
def test_encode_mistakes_are_caught(monkeypatch, bad):
    monkeypatch.setattr(pins_e4m3, "e4m3_encode", bad)
    with pytest.raises(AssertionError):
        pins_e4m3.test_encode_brute_force_midpoints_and_neighbours()


def _w8a8_scale_per_tile(xq, xs, wq, ws):
    """The latent bug the Ada post describes: one weight scale per tile."""
    M, K = xq.shape
    y = np.zeros((M, wq.shape[0]))
    for kb in range(K // BLK128):
        ks = slice(kb * BLK128, (kb + 1) * BLK128)
        y += (e4m3_decode(xq[:, ks]) @ e4m3_decode(wq[:, ks]).T) * xs[:, kb, None].astype(float) * float(ws[0, kb])
    return y


def _w8a8_drops_last_block(xq, xs, wq, ws):
    from oracle import gemm_w8a8_blk128
    K = xq.shape[1]
    return gemm_w8a8_blk128(xq[:, :K - BLK128], xs[:, :-1], wq[:, :K - BLK128], ws[:, :-1]) if K > BLK128 else 0 * gemm_w8a8_blk128(xq, xs, wq, ws)


@pytest.mark.parametrize("bad", [_w8a8_scale_per_tile, _w8a8_drops_last_block])
def test_w8a8_mistakes_are_caught(monkeypatch, bad):
    monkeypatch.setattr(pins_gemm, "gemm_w8a8_blk128", bad)
    with pytest.raises(AssertionError):
        pins_gemm.test_w8a8_exact_rational_bruteforce()


def _blk32_bias_off_by_one(x, wq, e8m0):
    from oracle import gemm_w8a16_blk32_ue8m0
    return gemm_w8a16_blk32_ue8m0(x, wq, e8m0) * 0.5


def test_blk32_mistake_is_caught(monkeypatch):
    monkeypatch.setattr(pins_gemm, "gemm_w8a16_blk32_ue8m0", _blk32_bias_off_by_one)
    with pytest.raises(AssertionError):
        pins_gemm.test_blk32_exact_rational()


def _dequant_transposed_scales(wq, scales, block):
    # scale of block (kb, nb) instead of (nb, kb): a plausible indexing slip
    wq = np.asarray(wq, np.uint8)
    N, K = wq.shape
    out = np.empty((N, K), np.float32)
    for n in range(N):
        for k in range(K):
            i, j = k // block, n // block
            s = scales[i, j] if i < scales.shape[0] and j < scales.shape[1] else scales[0, 0]
            out[n, k] = np.float32(e4m3_decode(wq[n, k])) * s
    return out


def _dequant_rounded_twice(wq, scales, block):
    # product formed in bf16 arithmetic (rounded operands) instead of one fp32 rounding
    from oracle import dequantize_weight, round_bf16
    return round_bf16(dequantize_weight(wq, round_bf16(scales), block))


@pytest.mark.parametrize("bad", [_dequant_transposed_scales, _dequant_rounded_twice])
def test_dequant_mistakes_are_caught(monkeypatch, bad):
    import tests.test_oracle_dequant as pins_dq
    monkeypatch.setattr(pins_dq, "dequantize_weight", bad)
    failures = 0
    for pin in (lambda: pins_dq.test_block_map(32, 96, 160), lambda: pins_dq.test_block_map(128, 200, 264),
                pins_dq.test_single_fp32_rounding, pins_dq.test_round_trip_of_the_weight_quantiser):
        try:
            pin()
        except AssertionError:
            failures += 1
    assert failures >= 1
