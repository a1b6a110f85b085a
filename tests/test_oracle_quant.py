"""Pins for the oracle's 1x128 activation and 128x128 weight quantisers.

Each group's scale is checked with exact rational arithmetic to be the
correctly rounded fp32 value of amax/448, each scaled element to be the
correctly rounded fp32 quotient x/s, and each code to be the brute-force
nearest E4M3 value of that quotient (ties to even, saturating).  Invariants the
construction fixes are checked too: the group maximum maps to +-448, negating
the input flips only the sign bits, zero groups give scale 0 and code 0, and a
ragged last group sees only its own columns.
"""

from fractions import Fraction

import numpy as np
import torch

from oracle import e4m3_decode, quantize_act_1x128, quantize_weight_128x128
from tests.test_oracle_e4m3 import _brute_force_encode


def _is_round_nearest_even_f32(f, exact):
    f = np.float32(f)
    d = abs(Fraction(float(f)) - exact)
    for nb in (np.nextafter(f, np.float32(-np.inf)), np.nextafter(f, np.float32(np.inf))):
        dn = abs(Fraction(float(nb)) - exact)
        if dn < d:
            return False
        if dn == d and (int(np.array(f).view(np.uint32)) & 1):
            return False
    return True


def _bf16(shape, seed, scale=1.0):
    z = np.random.default_rng(seed).standard_normal(shape).astype(np.float32) * np.float32(scale)
    return torch.from_numpy(z).to(torch.bfloat16).float().numpy()


def _check_group(vals, codes, s):
    vals = np.asarray(vals, np.float32)
    amax = float(np.max(np.abs(vals)))
    if amax == 0.0:
        assert s == 0.0 and np.all(codes == 0)
        return
    assert _is_round_nearest_even_f32(s, Fraction(amax) / 448)
    exact_q = [Fraction(float(v)) / Fraction(float(s)) for v in vals]
    # the correctly rounded fp32 quotient, found by search around the float64 quotient
    t = []
    for v, e in zip(vals, exact_q):
        c = np.float32(float(v) / float(s))
        for cand in (c, np.nextafter(c, np.float32(-np.inf)), np.nextafter(c, np.float32(np.inf))):
            if _is_round_nearest_even_f32(cand, e):
                t.append(cand)
                break
        else:
            raise AssertionError("no correctly rounded neighbour found")
    np.testing.assert_array_equal(codes, _brute_force_encode(np.array(t, np.float32)))


def test_act_quant_exact_rational_small():
    x = _bf16((3, 300), 7)                     # ragged: groups of 128, 128, 44
    x[1, 128:256] *= 0.0                       # a zero group
    xq, xs = quantize_act_1x128(x)
    assert xq.shape == (3, 300) and xs.shape == (3, 3) and xs.dtype == np.float32
    for m in range(3):
        for g in range(3):
            lo, hi = 128 * g, min(300, 128 * g + 128)
            _check_group(x[m, lo:hi], xq[m, lo:hi], xs[m, g])


def test_act_quant_invariants():
    x = _bf16((8, 1024), 11, scale=3.0)
    xq, xs = quantize_act_1x128(x)
    d = e4m3_decode(xq)
    for m in range(8):
        for g in range(8):
            grp = x[m, 128 * g:128 * g + 128]
            k = int(np.argmax(np.abs(grp)))
            assert abs(d[m, 128 * g + k]) == 448.0
            # reconstruction error: at most half an E4M3 step at the value, plus fp32 rounding
            s = float(xs[m, g])
            rec = d[m, 128 * g:128 * g + 128] * s
            step = np.where(np.abs(grp / s) < 2 ** -6, 2.0 ** -9,
                            np.exp2(np.floor(np.log2(np.maximum(np.abs(grp / s), 2 ** -6))) - 3))
            assert np.all(np.abs(rec - grp) <= (step / 2) * s * (1 + 1e-6) + 1e-30)
    xq_neg, xs_neg = quantize_act_1x128(-x)
    np.testing.assert_array_equal(xs_neg, xs)
    np.testing.assert_array_equal(xq_neg, xq ^ 0x80)


def test_act_quant_power_of_two_homogeneity():
    x = _bf16((2, 256), 5)
    xq, xs = quantize_act_1x128(x)
    xq2, xs2 = quantize_act_1x128(x * np.float32(2.0 ** 5))
    np.testing.assert_array_equal(xq2, xq)
    np.testing.assert_array_equal(xs2, xs * np.float32(2.0 ** 5))


def test_ragged_group_sees_only_its_columns():
    x = _bf16((1, 200), 3)
    x[0, 150] = 100.0                          # in the ragged group [128, 200)
    xq, xs = quantize_act_1x128(x)
    assert xs[0, 1] == np.float32(np.float32(100.0) / np.float32(448.0))
    assert xs[0, 0] == np.float32(np.max(np.abs(x[0, :128])) / np.float32(448.0))


def test_weight_quant_exact_rational_ragged():
    w = _bf16((200, 260), 21, scale=0.02)      # ragged in both directions
    wq, ws = quantize_weight_128x128(w)
    assert ws.shape == (2, 3)
    for nb in range(2):
        for kb in range(3):
            blk = w[128 * nb:128 * nb + 128, 128 * kb:128 * kb + 128]
            q = wq[128 * nb:128 * nb + 128, 128 * kb:128 * kb + 128]
            amax = float(np.max(np.abs(blk)))
            assert _is_round_nearest_even_f32(ws[nb, kb], Fraction(amax) / 448)
            # exact check of the codes on a sample of each tile's elements
            sample = np.random.default_rng(nb * 10 + kb).choice(blk.size, 64, replace=False)
            t = []
            for i in sample:
                v = blk.reshape(-1)[i]
                e = Fraction(float(v)) / Fraction(float(ws[nb, kb]))
                c = np.float32(float(v) / float(ws[nb, kb]))
                for cand in (c, np.nextafter(c, np.float32(-np.inf)), np.nextafter(c, np.float32(np.inf))):
                    if _is_round_nearest_even_f32(cand, e):
                        t.append(cand)
                        break
            np.testing.assert_array_equal(q.reshape(-1)[sample], _brute_force_encode(np.array(t, np.float32)))
