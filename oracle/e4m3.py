"""OCP E4M3 ("fn") decode and encode — oracle, test infrastructure only.

Format, as the pages state it ([ARC] "What this adds"; [SM70] "Exactness";
[3090] §4.1): one sign bit, four exponent bits with bias 7, three mantissa
bits.  Exponent field 0 holds the subnormals m * 2^-9.  Sign.1111.111 is NaN
and there is no infinity, so the largest finite magnitude is 1.75 * 2^8 = 448.
Every finite value is a multiple of 2^-9 with at most four significant bits.

Rounding mode and overflow are not stated on the pages.  The reading taken
here: round to nearest, ties to even, and saturate to +-448 (a quantiser that
divides by amax/448 can land a hair above 448 through fp32 rounding, and
saturation is the only choice that keeps the code finite).  The sign of zero
is kept (-0 encodes as 0x80).
"""

import numpy as np

E4M3_MAX = 448.0
E4M3_NAN_CODES = (0x7F, 0xFF)


def e4m3_decode(codes):
    """Exact value of each E4M3 code as float64 (NaN for 0x7F / 0xFF).

    Closed form: s = bit 7, E = bits 6..3, m = bits 2..0;
    E == 0 gives (-1)^s * m * 2^-9, otherwise (-1)^s * (1 + m/8) * 2^(E-7).
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = c >> 7
    E = (c >> 3) & 0xF
    m = c & 0x7
    subnormal = m * 2.0 ** -9
    normal = (1.0 + m / 8.0) * np.exp2((E - 7).astype(np.float64))
    mag = np.where(E == 0, subnormal, normal)
    val = np.where(s == 1, -mag, mag)
    return np.where((c & 0x7F) == 0x7F, np.nan, val)


def e4m3_encode(a):
    """E4M3 code of each fp32 value: round to nearest even, saturate to +-448.

    The input is taken as IEEE fp32 (it is the fp32 quotient the quantiser
    forms); it is widened exactly to float64 and every step below is exact in
    float64, so the only rounding is the one to E4M3.  NaN inputs are outside
    the domain.
    """
    a = np.asarray(a, dtype=np.float32).astype(np.float64)
    negative = np.signbit(a)
    mag = np.abs(a)

    # Subnormal range |a| < 2^-6: the code's mantissa is |a| in units of 2^-9.
    # A result of 8 units is 2^-6, whose code (E=1, m=0) is the integer 8 too.
    sub_units = np.rint(np.minimum(mag, 1.0) * 512.0)  # np.rint rounds half to even

    # Normal range: |a| = (1 + f) * 2^(E-7) with f in [0, 1).
    _, ex = np.frexp(np.where(mag > 0, mag, 1.0))  # mag = frac * 2^ex, frac in [0.5, 1)
    E = ex - 1 + 7
    mant = np.rint((mag / np.exp2((E - 7).astype(np.float64)) - 1.0) * 8.0)
    carry = mant == 8.0  # rounded up into the next binade
    E = np.where(carry, E + 1, E)
    mant = np.where(carry, 0.0, mant)
    normal_code = (E.astype(np.int64) << 3) | mant.astype(np.int64)

    code = np.where(mag < 2.0 ** -6, sub_units.astype(np.int64), normal_code)
    code = np.where(mag >= E4M3_MAX, 0x7E, code)
    code = np.where(negative, code | 0x80, code)
    return code.astype(np.uint8)
