"""Pins of the tolerance bar (oracle/compare.py), the check every GEMM parity
test goes through.

The bar (fixed for this path, not by the pages): against the float64 oracle
Y0, max |Y - Y0| <= 1e-2 * rms(Y0) with rms over all M*N outputs of Y0, and
||Y - Y0||_F / ||Y0||_F <= 4e-3.  For 16-bit outputs each element may also
carry half an ulp of the output format at |Y0| (round-to-nearest of a result
that already meets the fp32 bar).  The pins below fix every piece of that:
hand-computed values of the error measures, arrays built to sit just inside
and just outside each bound (pass must turn to fail), the half-ulp against the
spacing of the formats taken from their bit patterns, and rms taken over Y0,
not over Y."""

import numpy as np
import pytest

from oracle import gemm_error, check_gemm_fp32, check_gemm_16bit
from oracle.compare import _half_ulp


# ------------------------------------------------------- the error measures ----

def test_gemm_error_hand_computed():
    """y0 = [[3, 4]], y = [[3, 4.5]]: max |err| = 0.5, rms(y0) = sqrt(12.5),
    ||y0||_F = 5, so rel = 0.5 / 5 = 0.1 (all exact in binary)."""
    e = gemm_error(np.array([[3.0, 4.5]]), np.array([[3.0, 4.0]]))
    assert e["max_abs_err"] == 0.5
    assert e["rms_ref"] == np.sqrt(12.5)
    assert e["rel_frob"] == 0.1


def test_gemm_error_rms_is_over_the_reference():
    """A wild output must not inflate the yardstick: rms comes from y0."""
    y0 = np.ones((2, 2))
    y = np.array([[1.0, 1.0], [1.0, 101.0]])
    e = gemm_error(y, y0)
    assert e["rms_ref"] == 1.0
    assert e["max_abs_err"] == 100.0
    assert e["rel_frob"] == 100.0 / 2.0


def test_gemm_error_uses_the_largest_element_error():
    """The max is over every element (one large error among many small ones)."""
    y0 = np.zeros((3, 5)) + 2.0
    y = y0.copy()
    y[1, 3] += 0.25
    y[0, 0] -= 0.125
    y[2, 4] -= 0.5
    assert gemm_error(y, y0)["max_abs_err"] == 0.5


# ------------------------------------------------------- fp32 bar: both flips --

def _reference(seed=0, shape=(16, 24)):
    y0 = np.random.default_rng(seed).standard_normal(shape) * 3.0
    return y0, float(np.sqrt(np.mean(y0 * y0)))


@pytest.mark.parametrize("factor,ok", [(1 - 1e-6, True), (1 + 1e-6, False)])
def test_fp32_max_error_bound_flips(factor, ok):
    """One element off by 1e-2 * rms(y0) * (1 -/+ 1e-6); the relative error of
    a single element stays far below 4e-3, so only the max bound decides."""
    y0, rms = _reference(1)
    y = y0.copy()
    y[5, 7] += 1e-2 * rms * factor
    got, e = check_gemm_fp32(y, y0)
    assert e["rel_frob"] < 1e-3
    assert got is ok


@pytest.mark.parametrize("factor,ok", [(1 - 1e-6, True), (1 + 1e-6, False)])
def test_fp32_relative_bound_flips(factor, ok):
    """Every element off by +-c with c = 4e-3 * rms(y0) * (1 -/+ 1e-6): the
    relative Frobenius error is c / rms(y0) (||y0||_F = rms * sqrt(n)) while
    the max error c stays below 1e-2 * rms, so only the relative bound decides."""
    y0, rms = _reference(2)
    signs = np.where(np.random.default_rng(3).random(y0.shape) < 0.5, -1.0, 1.0)
    c = 4e-3 * rms * factor
    got, e = check_gemm_fp32(y0 + c * signs, y0)
    assert e["max_abs_err"] < 1e-2 * rms
    assert abs(e["rel_frob"] - c / rms) < 1e-12
    assert got is ok


def test_fp32_exact_result_passes():
    y0, _ = _reference(4)
    assert check_gemm_fp32(y0.copy(), y0)[0]


# --------------------------------------------------------------- half an ulp --

def _f16_spacing_from_bits(v):
    """Distance from the fp16 value v (|v| < 65504) to the next fp16 value up
    in magnitude, from the bit pattern (independent of frexp)."""
    h = np.abs(np.asarray(v, np.float16))
    nxt = (h.view(np.uint16) + np.uint16(1)).view(np.float16)
    return nxt.astype(np.float64) - h.astype(np.float64)


def _bf16_spacing_from_bits(v):
    """Same for bf16 values held exactly in float32 (low 16 bits zero)."""
    f = np.abs(np.asarray(v, np.float32))
    bits = f.view(np.uint32)
    assert np.all(bits & 0xFFFF == 0)
    nxt = (bits + np.uint32(0x10000)).view(np.float32)
    return nxt.astype(np.float64) - f.astype(np.float64)


def test_half_ulp_f16_every_finite_value():
    """Every positive finite fp16 value below the largest: normals and
    subnormals (spacing 2^-24), against np.spacing and the bit pattern."""
    bits = np.arange(1, 0x7BFF, dtype=np.uint16)
    v = bits.view(np.float16)
    want = _f16_spacing_from_bits(v) / 2
    np.testing.assert_array_equal(_half_ulp(v.astype(np.float64), 10, -14), want)
    np.testing.assert_array_equal(want, np.spacing(v).astype(np.float64) / 2)
    np.testing.assert_array_equal(_half_ulp(-v.astype(np.float64), 10, -14), want)


def test_half_ulp_bf16_normals_and_subnormals():
    """bf16 values of every exponent (normals and subnormals, spacing 2^-133)."""
    rng = np.random.default_rng(5)
    hi = rng.integers(1, 0x7F7F, size=20000, dtype=np.uint32)
    hi = np.concatenate([hi, np.arange(1, 0x100, dtype=np.uint32), np.array([0x0080, 0x3F80, 0x7F00], np.uint32)])
    v = (hi << 16).view(np.float32)
    want = _bf16_spacing_from_bits(v) / 2
    np.testing.assert_array_equal(_half_ulp(v.astype(np.float64), 7, -126), want)
    assert _half_ulp(np.array([2.0 ** -130]), 7, -126)[0] == 2.0 ** -134


def test_half_ulp_between_representable_values():
    """A float64 y0 between two 16-bit values takes the spacing of its own
    binade: RN of it is within that half spacing."""
    y0 = np.array([1.0 + 2.0 ** -9, 3.999, 1000.3, -0.7])
    np.testing.assert_array_equal(_half_ulp(y0, 7, -126), [2.0 ** -8, 2.0 ** -7, 2.0 ** 1, 2.0 ** -9])
    np.testing.assert_array_equal(_half_ulp(y0, 10, -14), [2.0 ** -11, 2.0 ** -10, 2.0 ** -2, 2.0 ** -12])


# ---------------------------------------------------------- 16-bit bar flips --

def _rne16(y, fmt):
    if fmt == "f16":
        return np.asarray(y, np.float64).astype(np.float16).astype(np.float64)
    f = np.asarray(y, np.float64).astype(np.float32).view(np.uint32).astype(np.uint64)
    r = ((f + 0x7FFF + ((f >> 16) & 1)) >> 16) << 16
    return r.astype(np.uint32).view(np.float32).astype(np.float64)


@pytest.mark.parametrize("fmt", ["bf16", "f16"])
def test_16bit_rounded_result_passes_where_the_bare_bar_fails(fmt):
    """RN(y0) to the 16-bit format passes the widened bar, while the bare fp32
    bar fails it (half an ulp of the large outputs exceeds 1e-2 * rms)."""
    rng = np.random.default_rng(6)
    y0 = rng.standard_normal((32, 64)) * 40.0
    y0[0, 0] = 4005.0                       # a large output, 5 from its bf16 neighbour 4000
    y = _rne16(y0, fmt)
    assert check_gemm_16bit(y, y0, fmt)[0]
    if fmt == "bf16":
        assert not check_gemm_fp32(y, y0)[0]


@pytest.mark.parametrize("fmt", ["bf16", "f16"])
def test_16bit_one_ulp_off_fails(fmt):
    """One large element a whole ulp away from RN(y0) fails: one ulp is more
    than 1e-2 * rms + half an ulp there."""
    rng = np.random.default_rng(7)
    y0 = rng.standard_normal((32, 64))
    y0[3, 9] = 250.0 + 2.0 ** -20
    y = _rne16(y0, fmt)
    ulp = 2.0 * _half_ulp(np.array([250.0]), 7 if fmt == "bf16" else 10, -126 if fmt == "bf16" else -14)[0]
    rms = float(np.sqrt(np.mean(y0 * y0)))
    assert ulp > 1e-2 * rms + ulp / 2
    assert check_gemm_16bit(y, y0, fmt)[0]
    y[3, 9] += ulp
    assert not check_gemm_16bit(y, y0, fmt)[0]


@pytest.mark.parametrize("fmt", ["bf16", "f16"])
@pytest.mark.parametrize("factor,ok", [(1 - 1e-6, True), (1 + 1e-6, False)])
def test_16bit_per_element_bound_flips(fmt, factor, ok):
    """y0 on a 16-bit value v; y = y0 + (1e-2 * rms + half ulp(v)) * (1 -/+ 1e-6)
    at one element (y itself need not be representable: the check takes the
    widened values as given)."""
    y0 = np.full((8, 8), 1.5)
    rms = 1.5
    y = y0.copy()
    h = _half_ulp(np.array([1.5]), 7 if fmt == "bf16" else 10, -126 if fmt == "bf16" else -14)[0]
    y[2, 2] += (1e-2 * rms + h) * factor
    assert check_gemm_16bit(y, y0, fmt)[0] is ok


@pytest.mark.parametrize("fmt", ["bf16", "f16"])
@pytest.mark.parametrize("factor,ok", [(1 - 1e-6, True), (1 + 1e-6, False)])
def test_16bit_relative_bound_flips(fmt, factor, ok):
    """The 16-bit check keeps the 4e-3 relative bound (same construction as
    the fp32 case, errors well inside the per-element bound)."""
    y0, rms = _reference(8)
    signs = np.where(np.random.default_rng(9).random(y0.shape) < 0.5, -1.0, 1.0)
    got, _ = check_gemm_16bit(y0 + 4e-3 * rms * factor * signs, y0, fmt)
    assert got is ok
