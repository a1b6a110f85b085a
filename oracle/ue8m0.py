"""Load-time validation of 32x32 power-of-two block scales — oracle, test
infrastructure only.

[SM70] "Exactness": an E4M3 value times 2^e is an exact FP16 value for every
e in [-14, 7], so a kernel that expands the weights to FP16 in registers
multiplies exactly the weights of a load-time FP16 dequantisation.  The packer
on that page refuses, loudly, (a) scales outside that window, (b) scales that
are not powers of two and (c) E4M3 NaN codes.

Reading taken for the order of checks and the reported index: every weight
code is checked first in row-major order, then every scale in row-major
order; the first failure found is reported with its flat index into the array
it belongs to.  A scale that is zero, negative, infinite or NaN is "not a
power of two".  A positive power of two 2^e outside [-14, 7] (including fp32
subnormal powers of two) is "outside the window".  Accepted scales are
emitted as the UE8M0 byte E = e + 127.
"""

import enum

import numpy as np

WINDOW = (-14, 7)


class Refusal(enum.Enum):
    OK = "ok"
    NAN_CODE = "nan_code"
    SCALE_NOT_POW2 = "scale_not_pow2"
    SCALE_WINDOW = "scale_window"


def prepare_blk32_ue8m0(wq, scale):
    """Validate wq [N,K] u8 and scale [N/32, K/32] f32.

    Returns (Refusal, e8m0 bytes or None, bad flat index or -1).
    """
    wq = np.asarray(wq, dtype=np.uint8)
    scale = np.asarray(scale, dtype=np.float32)
    N, K = wq.shape
    assert N % 32 == 0 and K % 32 == 0 and scale.shape == (N // 32, K // 32)

    flat_codes = wq.reshape(-1)
    bad = np.flatnonzero((flat_codes & 0x7F) == 0x7F)
    if bad.size:
        return Refusal.NAN_CODE, None, int(bad[0])

    out = np.zeros(scale.shape, dtype=np.uint8)
    flat_scale = scale.reshape(-1)
    flat_out = out.reshape(-1)
    for i, s in enumerate(flat_scale.astype(np.float64)):
        if not np.isfinite(s) or s <= 0.0:
            return Refusal.SCALE_NOT_POW2, None, i
        frac, ex = np.frexp(s)          # s = frac * 2^ex exactly, frac in [0.5, 1)
        if frac != 0.5:
            return Refusal.SCALE_NOT_POW2, None, i
        e = int(ex) - 1
        if not (WINDOW[0] <= e <= WINDOW[1]):
            return Refusal.SCALE_WINDOW, None, i
        flat_out[i] = e + 127
    return Refusal.OK, out, -1
