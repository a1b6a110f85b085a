"""The seeded input generators shared by the tests and the bench (CPU only):
reproducible per (workload, stream), and drawing the value sets their
docstrings state."""

import numpy as np
import torch

from blockwise_scaled_fp8_amd import inputs

FINITE = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)


def test_draws_are_reproducible_per_workload_and_stream():
    a = inputs.e4m3_codes(3, 1024, 5, 2)
    assert torch.equal(a, inputs.e4m3_codes(3, 1024, 5, 2))
    assert not torch.equal(a, inputs.e4m3_codes(3, 1024, 5, 3))
    assert not torch.equal(a, inputs.e4m3_codes(3, 1024, 6, 2))
    x = inputs.activations(4, 512, 0)
    assert torch.equal(x, inputs.activations(4, 512, 0)) and x.dtype == torch.bfloat16


def test_e4m3_codes_cover_exactly_the_finite_codes():
    v = inputs.e4m3_codes(64, 4096, 5, 0).numpy()
    assert v.dtype == np.uint8 and v.shape == (64, 4096)
    np.testing.assert_array_equal(np.unique(v), FINITE)         # all 254, no NaN code
    counts = np.bincount(v.ravel(), minlength=256)[FINITE]
    assert counts.min() > 0.8 * v.size / 254 and counts.max() < 1.2 * v.size / 254   # about 6 sigma


def test_block_scales_positive_in_their_range():
    s = inputs.block_scales(7, 300, 5, 1).numpy()
    assert s.dtype == np.float32 and s.shape == (7, 300)
    assert (s >= np.float32(2.0 ** -10)).all() and (s < np.float32(2.0 ** -4) * (1 + 2 ** -20)).all()
    e = np.log2(s.astype(np.float64))
    assert e.min() < -9.5 and e.max() > -4.5                     # spans the range


def test_block32_scales_are_powers_of_two_in_the_window():
    s = inputs.block32_scales(64, 1024, 3, lo=-14, hi=7).numpy()
    frac, ex = np.frexp(s)
    assert (frac == 0.5).all()
    assert set(np.unique(ex - 1)) == set(range(-14, 8))


def test_outlier_columns():
    K = 4096
    plain = inputs.activations(2, K, 9, stream=0).float()
    out = inputs.activations(2, K, 9, stream=0, outliers=True).float()
    changed = (plain != out).any(dim=0).nonzero().flatten()
    assert len(changed) <= int(np.ceil(0.01 * K)) and len(changed) >= int(np.ceil(0.01 * K)) - 2
    ratio = (out[:, changed] / plain[:, changed]).abs()
    assert ((ratio > 19) & (ratio < 21)).all()


def test_workload_shapes():
    assert inputs.workload(0)["x"].shape == (4, 512) and inputs.workload(0)["w"].shape == (512, 512)
    w1 = inputs.workload(1)
    assert w1["x"].shape == (1, 4096) and w1["w"].shape == (4096, 4096)
    assert inputs.workload(2, M=8)["x"].shape == (8, 4096)
    w = w1["w"].float()
    assert abs(w.std().item() - inputs.W_SIGMA) < 1e-3
