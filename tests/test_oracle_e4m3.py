"""Pins for the oracle's E4M3 decode and encode.

Decode is pinned three independent ways against the closed form: the integer
identity on the block-32 model card ([SM70] "How it works": the byte's seven
magnitude bits shifted into an FP16 word give the value times 2^-8), its
fp32 analogue (bias difference 2^120, [3090] §4.1), and torch's float8_e4m3fn
type; plus the format facts the pages state ([SM70] "Exactness").
Encode is pinned by a brute-force nearest-value search over the 253 finite
values with ties to the even code, over random fp32 values and over every
midpoint and its fp32 neighbours, and by torch's cast where it is defined.
"""

import numpy as np
import pytest
import torch

from oracle import e4m3_decode, e4m3_encode

ALL = np.arange(256, dtype=np.uint8)
FINITE = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)


def test_decode_matches_fp16_integer_identity():
    b = FINITE.astype(np.uint16)
    bits = ((b & 0x7F) << 7) | ((b & 0x80) << 8)
    via_fp16 = bits.astype(np.uint16).view(np.float16).astype(np.float64) * 2.0 ** 8
    np.testing.assert_array_equal(via_fp16, e4m3_decode(FINITE))
    # the sign of zero survives both routes
    assert np.signbit(e4m3_decode(np.uint8(0x80)))


def test_decode_matches_fp32_bias_120_identity():
    b = FINITE.astype(np.uint32)
    bits = ((b & 0x7F) << 20) | ((b & 0x80) << 24)
    via_fp32 = bits.view(np.float32).astype(np.float64) * 2.0 ** 120
    np.testing.assert_array_equal(via_fp32, e4m3_decode(FINITE))


def test_decode_matches_torch_float8_e4m3fn():
    t = torch.from_numpy(ALL.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    d = e4m3_decode(ALL)
    assert np.array_equal(np.isnan(t), np.isnan(d))
    np.testing.assert_array_equal(t[~np.isnan(t)], d[~np.isnan(d)])


def test_decode_format_facts():
    d = e4m3_decode(ALL)
    nan_codes = [int(c) for c in ALL if np.isnan(d[c])]
    assert nan_codes == [0x7F, 0xFF]
    fin = d[~np.isnan(d)]
    assert fin.size == 254
    assert np.unique(fin).size == 253           # +0 and -0 coincide
    assert fin.max() == 448.0 and fin.min() == -448.0
    assert fin[fin > 0].min() == 2.0 ** -9
    # multiples of 2^-9 with at most four significant bits
    units = fin * 2 ** 9
    assert np.all(units == np.round(units))
    for u in np.abs(units[units != 0]).astype(np.int64):
        while u % 2 == 0:
            u //= 2
        assert u < 16
    # exactly representable in fp16 after the 2^-8 shift and in bf16
    assert np.all(fin.astype(np.float16).astype(np.float64) == fin)
    assert np.all(torch.from_numpy(fin).to(torch.bfloat16).to(torch.float64).numpy() == fin)


# ---------------------------------------------------------------- encode ----

_POS_CODES = np.array([c for c in range(0x7F)], dtype=np.uint8)    # 0x00..0x7E
_POS_VALUES = e4m3_decode(_POS_CODES)


def _brute_force_encode(a):
    """Nearest finite E4M3 value by exhaustive search, ties to the code whose
    mantissa LSB is 0, magnitudes >= 448 saturated; sign kept."""
    out = np.empty(a.shape, dtype=np.uint8)
    for i, v in enumerate(np.asarray(a, np.float32).astype(np.float64).reshape(-1)):
        mag = abs(v)
        if mag >= 448.0:
            code = 0x7E
        else:
            dist = np.abs(_POS_VALUES - mag)
            best = np.flatnonzero(dist == dist.min())
            if best.size > 1:
                best = [c for c in best if (_POS_CODES[c] & 1) == 0]
            code = int(_POS_CODES[best[0]])
        out.reshape(-1)[i] = code | (0x80 if np.signbit(v) else 0)
    return out


def test_encode_roundtrip_all_finite_codes():
    np.testing.assert_array_equal(e4m3_encode(e4m3_decode(FINITE).astype(np.float32)), FINITE)


def test_encode_brute_force_random():
    g = np.random.default_rng(1234)
    a = np.concatenate([
        g.standard_normal(20000).astype(np.float32) * 60,
        (g.standard_normal(5000) * 2.0 ** -7).astype(np.float32),   # subnormal range
        g.uniform(-470, 470, 5000).astype(np.float32),             # saturation edge
    ])
    np.testing.assert_array_equal(e4m3_encode(a), _brute_force_encode(a))


def test_encode_brute_force_midpoints_and_neighbours():
    v = np.sort(np.unique(_POS_VALUES))
    mids = ((v[:-1] + v[1:]) / 2).astype(np.float32)
    assert np.all(mids.astype(np.float64) == (v[:-1] + v[1:]) / 2)   # midpoints are exact fp32
    pts = np.concatenate([mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(1000)),
                          np.float32([448.0, 456.0, 464.0, 465.0, 1e6, 3e38])])
    pts = np.concatenate([pts, -pts])
    np.testing.assert_array_equal(e4m3_encode(pts), _brute_force_encode(pts))


def test_encode_agrees_with_torch_cast_inside_range():
    g = np.random.default_rng(99)
    a = np.concatenate([g.uniform(-448, 448, 50000), g.standard_normal(50000) * 2.0 ** -8]).astype(np.float32)
    ref = torch.from_numpy(a).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(e4m3_encode(a), ref)


@pytest.mark.parametrize("value,code", [
    (464.0, 0x7E), (1e9, 0x7E), (-1e9, 0xFE), (448.0, 0x7E),
    (-0.0, 0x80), (0.0, 0x00), (2.0 ** -10, 0x00), (3 * 2.0 ** -10, 0x02),
    (-1e-9, 0x80), (1.0, 0x38), (-2.0, 0xC0), (2.0 ** -6, 0x08), (15 * 2.0 ** -10, 0x08),
])
def test_encode_special_values(value, code):
    assert int(e4m3_encode(np.float32(value))) == code
