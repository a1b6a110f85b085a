"""Pins for the oracle's three block-scaled products and the block-32 validator.

W8A8 and W8A16 blk128 are checked against exact rational arithmetic on small
non-square shapes with distinct per-tile scales (a transposed operand, a
wrong scale index or a dropped block fails), against a plain float64 matmul
with unit scales (exact for these sizes), against one-hot inputs, and against
power-of-two scale homogeneity.  Block-32 is checked by the one-hot sweep of
all 254 finite codes times all 22 window exponents, which the block-32 model
card ([SM70] "Exactness") says is exact in FP16, and against exact rationals.
The validator is checked on every refusal class the model card lists.
"""

from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import (e4m3_decode, gemm_w8a8_blk128, gemm_w8a16_blk128, gemm_w8a16_blk32_ue8m0,
                    prepare_blk32_ue8m0, Refusal)

FINITE = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)


def _codes(shape, seed):
    return np.random.default_rng(seed).choice(FINITE, size=shape)


def _scales(shape, seed):
    g = np.random.default_rng(seed)
    return (g.uniform(0.5, 2.0, shape) * np.exp2(g.integers(-12, 4, shape))).astype(np.float32)


def _units(codes):
    """E4M3 values as exact integers in units of 2^-9."""
    u = e4m3_decode(codes) * 512.0
    assert np.all(u == np.round(u))
    return u.astype(np.int64)


def test_w8a8_exact_rational_bruteforce():
    M, N, K = 3, 320, 256          # three weight-scale rows (the last partial), two K blocks
    xq, wq = _codes((M, K), 1), _codes((N, K), 2)
    xs, ws = _scales((M, 2), 3), _scales((3, 2), 4)
    y = gemm_w8a8_blk128(xq, xs, wq, ws)
    ux, uw = _units(xq), _units(wq)
    for m in range(M):
        for n in range(N):
            exact, magnitude = Fraction(0), Fraction(0)
            for kb in range(2):
                p = int(np.dot(ux[m, 128 * kb:128 * kb + 128], uw[n, 128 * kb:128 * kb + 128]))
                term = Fraction(float(xs[m, kb])) * Fraction(float(ws[n // 128, kb])) * Fraction(p, 2 ** 18)
                exact += term
                magnitude += abs(term)
            # float64 promotion: a few roundings, each relative to the terms' magnitude
            assert abs(Fraction(float(y[m, n])) - exact) <= magnitude * Fraction(1, 2 ** 50)


def test_w8a8_unit_scales_equal_plain_matmul():
    M, N, K = 5, 256, 4096
    xq, wq = _codes((M, K), 5), _codes((N, K), 6)
    y = gemm_w8a8_blk128(xq, np.ones((M, 32), np.float32), wq, np.ones((2, 32), np.float32))
    np.testing.assert_array_equal(y, e4m3_decode(xq) @ e4m3_decode(wq).T)


def test_w8a8_one_hot():
    M, N, K = 4, 384, 512
    wq = _codes((N, K), 7)
    for k in (0, 127, 128, 511):
        xq = np.zeros((M, K), np.uint8)
        xq[:, k] = 0x38                          # 1.0
        y = gemm_w8a8_blk128(xq, np.ones((M, 4), np.float32), wq, np.ones((3, 4), np.float32))
        np.testing.assert_array_equal(y, np.broadcast_to(e4m3_decode(wq[:, k]), (M, N)))


def test_w8a8_scale_homogeneity_per_column_block():
    M, N, K = 2, 384, 256
    xq, wq = _codes((M, K), 8), _codes((N, K), 9)
    xs, ws = _scales((M, 2), 10), _scales((3, 2), 11)
    y = gemm_w8a8_blk128(xq, xs, wq, ws)
    ws2 = ws.copy()
    ws2[1, :] *= 2                               # weight rows 128..255 only
    y2 = gemm_w8a8_blk128(xq, xs, wq, ws2)
    np.testing.assert_array_equal(y2[:, 128:256], 2 * y[:, 128:256])
    np.testing.assert_array_equal(y2[:, :128], y[:, :128])
    np.testing.assert_array_equal(y2[:, 256:], y[:, 256:])
    xs2 = xs.copy()
    xs2[1, 1] *= 0.5                             # token 1, second K block only
    y3 = gemm_w8a8_blk128(xq, xs2, wq, ws)
    np.testing.assert_array_equal(y3[0], y[0])
    assert not np.array_equal(y3[1], y[1])


def test_w8a8_scale_once_equals_scale_per_slice_in_exact_arithmetic():
    """The per-32-slice promotion that spills on Ada and the once-per-block
    promotion are the same number in exact arithmetic ([ADA] "Where the
    registers went" / "The fix"); the oracle sits within float64 rounding of
    both."""
    xq, wq = _codes((1, 128), 12), _codes((16, 128), 13)
    xs, ws = _scales((1, 1), 14), _scales((1, 1), 15)
    y = gemm_w8a8_blk128(xq, xs, wq, ws)
    ux, uw = _units(xq), _units(wq)
    s = Fraction(float(xs[0, 0])) * Fraction(float(ws[0, 0]))
    for n in range(16):
        per_slice = sum(s * Fraction(int(np.dot(ux[0, j:j + 32], uw[n, j:j + 32])), 2 ** 18) for j in range(0, 128, 32))
        assert abs(Fraction(float(y[0, n])) - per_slice) <= abs(per_slice) * Fraction(1, 2 ** 51)


def _bf16(shape, seed):
    z = np.random.default_rng(seed).standard_normal(shape).astype(np.float32)
    return torch.from_numpy(z).to(torch.bfloat16).float().numpy()


def test_w8a16_blk128_exact_rational_bruteforce():
    M, N, K = 2, 272, 256
    x, wq, ws = _bf16((M, K), 16), _codes((N, K), 17), _scales((3, 2), 18)
    y = gemm_w8a16_blk128(x, wq, ws)
    d = e4m3_decode(wq)
    for m in range(M):
        for n in range(N):
            exact, magnitude = Fraction(0), Fraction(0)
            for kb in range(2):
                prods = [Fraction(float(x[m, k])) * Fraction(float(d[n, k])) for k in range(128 * kb, 128 * kb + 128)]
                exact += Fraction(float(ws[n // 128, kb])) * sum(prods)
                magnitude += Fraction(float(ws[n // 128, kb])) * sum(abs(p) for p in prods)
            assert abs(Fraction(float(y[m, n])) - exact) <= magnitude * Fraction(1, 2 ** 45)


def test_w8a16_blk128_one_hot():
    N, K = 256, 384
    wq, ws = _codes((N, K), 19), _scales((2, 3), 20)
    for k in (0, 200, 383):
        x = np.zeros((1, K), np.float32)
        x[0, k] = 1.0
        y = gemm_w8a16_blk128(x, wq, ws)
        np.testing.assert_array_equal(y[0], e4m3_decode(wq[:, k]) * ws[np.arange(N) // 128, k // 128].astype(np.float64))


def test_blk32_one_hot_all_codes_all_exponents_exact_in_fp16():
    """Every finite code times every window exponent, one output each."""
    exps = np.arange(-14, 8)
    N = 32 * exps.size                          # one 32-row tile per exponent
    K = 256                                     # 254 codes + 2 zero columns
    wq = np.zeros((N, K), np.uint8)
    wq[:, :254] = FINITE[None, :]
    e8 = np.repeat((exps + 127).astype(np.uint8)[:, None], K // 32, axis=1)
    d = e4m3_decode(FINITE)
    for k in range(254):
        x = np.zeros((1, K), np.float32)
        x[0, k] = 1.0
        y = gemm_w8a16_blk32_ue8m0(x, wq, e8)[0].reshape(exps.size, 32)
        expect = d[k] * np.exp2(exps.astype(np.float64))
        np.testing.assert_array_equal(y, np.repeat(expect[:, None], 32, axis=1))
        # the window claim: each scaled weight is an exact fp16 value
        assert np.all(expect.astype(np.float16).astype(np.float64) == expect)
    # just outside the window it is not exact any more (overflow at 2^8, lost bits at 2^-16)
    assert 448.0 * 2.0 ** 8 > float(np.finfo(np.float16).max)
    assert float(np.float16(2.0 ** -9 * 2.0 ** -16)) != 2.0 ** -25


def test_blk32_exact_rational():
    M, N, K = 2, 64, 96
    x, wq = _bf16((M, K), 22), _codes((N, K), 23)
    e8 = np.random.default_rng(24).integers(113, 135, size=(2, 3)).astype(np.uint8)
    y = gemm_w8a16_blk32_ue8m0(x, wq, e8)
    d = e4m3_decode(wq)
    for m in range(M):
        for n in range(N):
            prods = [Fraction(float(x[m, k])) * Fraction(float(d[n, k])) * Fraction(2) ** (int(e8[n // 32, k // 32]) - 127)
                     for k in range(K)]
            exact, magnitude = sum(prods), sum(abs(p) for p in prods)
            assert abs(Fraction(float(y[m, n])) - exact) <= magnitude * Fraction(1, 2 ** 45)


def test_oracle_refuses_nan_operands():
    with pytest.raises(ValueError):
        gemm_w8a8_blk128(np.full((1, 128), 0x7F, np.uint8), np.ones((1, 1), np.float32),
                         np.zeros((16, 128), np.uint8), np.ones((1, 1), np.float32))


# ------------------------------------------------------------- validator ----

def _valid(N=64, K=64):
    return _codes((N, K), 30), np.full((N // 32, K // 32), 1.0, np.float32)


def test_prepare_accepts_window_and_emits_biased_exponent():
    wq, s = _valid()
    s[0, 0], s[0, 1], s[1, 0], s[1, 1] = 2.0 ** -14, 2.0 ** 7, 1.0, 0.5
    st, e8, bad = prepare_blk32_ue8m0(wq, s)
    assert st is Refusal.OK and bad == -1
    np.testing.assert_array_equal(e8, np.array([[113, 134], [127, 126]], np.uint8))


@pytest.mark.parametrize("value,reason", [
    (3.0, Refusal.SCALE_NOT_POW2), (0.0, Refusal.SCALE_NOT_POW2), (-1.0, Refusal.SCALE_NOT_POW2),
    (-0.5, Refusal.SCALE_NOT_POW2), (np.inf, Refusal.SCALE_NOT_POW2), (np.nan, Refusal.SCALE_NOT_POW2),
    (1.5 * 2.0 ** -20, Refusal.SCALE_NOT_POW2),
    (2.0 ** -15, Refusal.SCALE_WINDOW), (2.0 ** 8, Refusal.SCALE_WINDOW), (2.0 ** -130, Refusal.SCALE_WINDOW),
    (2.0 ** 100, Refusal.SCALE_WINDOW),
])
def test_prepare_refuses_bad_scales(value, reason):
    wq, s = _valid()
    s[1, 0] = value
    st, e8, bad = prepare_blk32_ue8m0(wq, s)
    assert st is reason and e8 is None and bad == 2


@pytest.mark.parametrize("code", [0x7F, 0xFF])
def test_prepare_refuses_nan_codes_first(code):
    wq, s = _valid()
    wq[3, 5] = code
    wq[10, 1] = code
    s[0, 0] = 3.0                                  # a bad scale too: codes are checked first
    st, e8, bad = prepare_blk32_ue8m0(wq, s)
    assert st is Refusal.NAN_CODE and bad == 3 * 64 + 5
