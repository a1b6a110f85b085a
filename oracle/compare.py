"""Tolerance bar for GEMM parity — test infrastructure only.

The bar for floating-point outputs (GEMM results are not unique: they depend
on the fp32 accumulation order) is, against the float64 oracle Y0:
    max |Y - Y0| <= 1e-2 * rms(Y0)      rms over all M*N outputs
    ||Y - Y0||_F / ||Y0||_F <= 4e-3
This bar is applied to the fp32-output mode, which is the same kernel and the
same accumulation as the 16-bit modes.

A 16-bit output cannot meet the max-error bar on its own for large outputs:
one bf16 ulp at |y| >= 2^e is 2^(e-7), which exceeds 1e-2 * rms as soon as
|y| is a few times the rms.  For 16-bit outputs the bar is therefore
    ||Y - Y0||_F / ||Y0||_F <= 4e-3  and, per element,
    |Y - Y0| <= 1e-2 * rms(Y0) + ulp16(Y0) / 2,
which any correctly accumulated, once-rounded result satisfies; and the
16-bit output must equal round-to-nearest-even of the kernel's own fp32
result bit for bit (checked by the tests with a library cast).
"""

import numpy as np

MAX_ERR_FRAC_OF_RMS = 1e-2
REL_FROB = 4e-3


def gemm_error(y, y0):
    y = np.asarray(y, dtype=np.float64)
    y0 = np.asarray(y0, dtype=np.float64)
    diff = y - y0
    rms = float(np.sqrt(np.mean(y0 * y0))) if y0.size else 0.0
    nrm = float(np.linalg.norm(y0))
    return {
        "max_abs_err": float(np.max(np.abs(diff))) if diff.size else 0.0,
        "rms_ref": rms,
        "rel_frob": float(np.linalg.norm(diff)) / nrm if nrm > 0 else float(np.linalg.norm(diff)),
    }


def check_gemm_fp32(y, y0):
    e = gemm_error(y, y0)
    ok = e["max_abs_err"] <= MAX_ERR_FRAC_OF_RMS * e["rms_ref"] and e["rel_frob"] <= REL_FROB
    return ok, e


def _half_ulp(y0, mant_bits, min_exp):
    """Half an ulp of the 16-bit format at |y0| (mant_bits explicit mantissa
    bits, min_exp the smallest normal exponent)."""
    a = np.abs(np.asarray(y0, np.float64))
    _, ex = np.frexp(np.where(a > 0, a, 1.0))
    e = np.maximum(ex - 1, min_exp)
    return np.exp2((e - mant_bits).astype(np.float64)) / 2.0


def check_gemm_16bit(y, y0, fmt):
    """fmt: 'bf16' or 'f16'.  y holds the 16-bit outputs widened exactly."""
    mant_bits, min_exp = {"bf16": (7, -126), "f16": (10, -14)}[fmt]
    e = gemm_error(y, y0)
    bound = MAX_ERR_FRAC_OF_RMS * e["rms_ref"] + _half_ulp(y0, mant_bits, min_exp)
    elem_ok = bool(np.all(np.abs(np.asarray(y, np.float64) - np.asarray(y0, np.float64)) <= bound))
    ok = elem_ok and e["rel_frob"] <= REL_FROB
    return ok, e
