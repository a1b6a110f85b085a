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


# ------------------------------------------------------- the tolerance bar ----

def _error_rms_over_output(y, y0):
    from oracle import gemm_error
    e = gemm_error(y, y0)
    e["rms_ref"] = float(np.sqrt(np.mean(np.asarray(y, np.float64) ** 2)))
    return e


def _error_rel_over_output(y, y0):
    from oracle import gemm_error
    e = gemm_error(y, y0)
    d = np.asarray(y, np.float64) - np.asarray(y0, np.float64)
    e["rel_frob"] = float(np.linalg.norm(d)) / float(np.linalg.norm(np.asarray(y, np.float64)))
    return e


def _error_mean_not_max(y, y0):
    from oracle import gemm_error
    e = gemm_error(y, y0)
    e["max_abs_err"] = float(np.mean(np.abs(np.asarray(y, np.float64) - np.asarray(y0, np.float64))))
    return e


@pytest.mark.parametrize("bad", [_error_rms_over_output, _error_rel_over_output, _error_mean_not_max])
def test_error_measure_mistakes_are_caught(monkeypatch, bad):
    import tests.test_oracle_compare as pins_cmp
    monkeypatch.setattr(pins_cmp, "gemm_error", bad)
    failures = 0
    for pin in (pins_cmp.test_gemm_error_hand_computed, pins_cmp.test_gemm_error_rms_is_over_the_reference,
                pins_cmp.test_gemm_error_uses_the_largest_element_error):
        try:
            pin()
        except AssertionError:
            failures += 1
    assert failures >= 1


def _fp32_bar_constants(max_frac, rel):
    def check(y, y0):
        from oracle import gemm_error
        e = gemm_error(y, y0)
        return e["max_abs_err"] <= max_frac * e["rms_ref"] and e["rel_frob"] <= rel, e
    return check


@pytest.mark.parametrize("bad", [_fp32_bar_constants(1e-3, 4e-3), _fp32_bar_constants(2e-2, 4e-3),
                                 _fp32_bar_constants(1e-2, 4e-2), _fp32_bar_constants(1e-2, 2e-3)])
def test_fp32_bar_constant_mistakes_are_caught(monkeypatch, bad):
    import tests.test_oracle_compare as pins_cmp
    monkeypatch.setattr(pins_cmp, "check_gemm_fp32", bad)
    failures = 0
    for factor, ok in ((1 - 1e-6, True), (1 + 1e-6, False)):
        for pin in (pins_cmp.test_fp32_max_error_bound_flips, pins_cmp.test_fp32_relative_bound_flips):
            try:
                pin(factor, ok)
            except AssertionError:
                failures += 1
    assert failures >= 1


def _half_ulp_full_ulp(y0, mant_bits, min_exp):
    from oracle.compare import _half_ulp
    return 2.0 * _half_ulp(y0, mant_bits, min_exp)


def _half_ulp_no_subnormal_floor(y0, mant_bits, min_exp):
    a = np.abs(np.asarray(y0, np.float64))
    _, ex = np.frexp(np.where(a > 0, a, 1.0))
    return np.exp2((ex - 1 - mant_bits).astype(np.float64)) / 2.0


def _half_ulp_exponent_off_by_one(y0, mant_bits, min_exp):
    from oracle.compare import _half_ulp
    return _half_ulp(y0, mant_bits - 1, min_exp)


@pytest.mark.parametrize("bad", [_half_ulp_full_ulp, _half_ulp_no_subnormal_floor, _half_ulp_exponent_off_by_one])
def test_half_ulp_mistakes_are_caught(monkeypatch, bad):
    import tests.test_oracle_compare as pins_cmp
    monkeypatch.setattr(pins_cmp, "_half_ulp", bad)
    failures = 0
    for pin in (pins_cmp.test_half_ulp_f16_every_finite_value, pins_cmp.test_half_ulp_bf16_normals_and_subnormals,
                pins_cmp.test_half_ulp_between_representable_values):
        try:
            pin()
        except AssertionError:
            failures += 1
    assert failures >= 1


def _16bit_without_half_ulp(y, y0, fmt):
    from oracle import check_gemm_fp32
    return check_gemm_fp32(y, y0)


def _16bit_without_relative_bound(y, y0, fmt):
    from oracle import gemm_error
    from oracle.compare import _half_ulp
    mant_bits, min_exp = {"bf16": (7, -126), "f16": (10, -14)}[fmt]
    e = gemm_error(y, y0)
    bound = 1e-2 * e["rms_ref"] + _half_ulp(y0, mant_bits, min_exp)
    return bool(np.all(np.abs(np.asarray(y, np.float64) - np.asarray(y0, np.float64)) <= bound)), e


def _16bit_formats_swapped(y, y0, fmt):
    from oracle import check_gemm_16bit
    return check_gemm_16bit(y, y0, "f16" if fmt == "bf16" else "bf16")


@pytest.mark.parametrize("bad", [_16bit_without_half_ulp, _16bit_without_relative_bound, _16bit_formats_swapped])
def test_16bit_bar_mistakes_are_caught(monkeypatch, bad):
    import tests.test_oracle_compare as pins_cmp
    monkeypatch.setattr(pins_cmp, "check_gemm_16bit", bad)
    failures = 0
    pins = [lambda fmt=fmt: pins_cmp.test_16bit_rounded_result_passes_where_the_bare_bar_fails(fmt)
            for fmt in ("bf16", "f16")]
    pins += [lambda fmt=fmt: pins_cmp.test_16bit_one_ulp_off_fails(fmt) for fmt in ("bf16", "f16")]
    pins += [lambda fmt=fmt, f=f, ok=ok: pins_cmp.test_16bit_per_element_bound_flips(fmt, f, ok)
             for fmt in ("bf16", "f16") for f, ok in ((1 - 1e-6, True), (1 + 1e-6, False))]
    pins += [lambda fmt=fmt, f=f, ok=ok: pins_cmp.test_16bit_relative_bound_flips(fmt, f, ok)
             for fmt in ("bf16", "f16") for f, ok in ((1 - 1e-6, True), (1 + 1e-6, False))]
    for pin in pins:
        try:
            pin()
        except AssertionError:
            failures += 1
    assert failures >= 1
