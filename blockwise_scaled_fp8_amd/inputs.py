"""Seeded synthetic inputs shared by the tests and the bench.

This module only draws random numbers and stores them in the input dtypes;
it holds none of the method's arithmetic (no block maxima, no scales, no
E4M3 rounding of the method's own).  Every draw comes from
``numpy.random.default_rng([workload_id, stream_id])`` so that each operand of
each workload is reproducible on its own.  fp32 draws become bf16 or fp16 by
torch's round-to-nearest-even cast.

Workloads (the shapes and value distributions of the pages' problems):
  0  W8A8 parity case: X [4, 512] ~ N(0, 1) bf16, W [512, 512] ~ N(0, 0.02^2) bf16
  1  o_proj decode:    X [1, 4096] ~ N(0, 1) bf16, W [4096, 4096] ~ N(0, 0.02^2) bf16
  2  o_proj prefill:   X [4096, 4096] ~ N(0, 1), 1% of the channels (41 columns,
                       chosen by a seeded permutation, the same for every token)
                       multiplied by 20 before the bf16 cast; W as workload 1
  3  block-32 weights: x [M, 7168] ~ N(0, 1) fp16; weight codes are the E4M3
                       codes of z ~ N(0, 1) [4096, 7168] (torch's float8_e4m3fn
                       cast; |z| never reaches 448 here); one power-of-two
                       scale 2^e per 32x32 tile, e uniform on {-14, ..., 7}
  4  projection sweep: W8A8 like workload 0 for (N, K) in {4096x4096, 1024x4096,
                       12288x4096, 4096x12288}
  5  longest K (2^23, the calls' limit), a few rows: E4M3 codes drawn
                       uniformly from the 254 finite codes for both operands,
                       fp32 block scales 2^u with u uniform on [-10, -4),
                       16-bit activations ~ N(0, 1) (drawn as codes and scales
                       directly: the 16-bit matrices and their quantisation
                       would take tens of GB on the host)
"""

import numpy as np
import torch

W_SIGMA = 0.02
OUTLIER_FRACTION = 0.01
OUTLIER_GAIN = 20.0

SWEEP_SHAPES = ((4096, 4096), (1024, 4096), (12288, 4096), (4096, 12288))
SWEEP_M = (1, 2, 4, 8, 16, 32, 64, 128, 512, 4096)


def rng(workload, stream):
    return np.random.default_rng([int(workload), int(stream)])


def normal(shape, workload, stream, sigma=1.0, dtype=torch.bfloat16):
    z = rng(workload, stream).standard_normal(size=shape, dtype=np.float32)
    if sigma != 1.0:
        z = z * np.float32(sigma)
    return torch.from_numpy(z).to(dtype)


def activations(M, K, workload, stream=0, outliers=False, dtype=torch.bfloat16):
    """X [M, K]; with outliers=True, ceil(1% of K) columns are scaled by 20
    before the cast to the 16-bit type."""
    z = rng(workload, stream).standard_normal(size=(M, K), dtype=np.float32)
    if outliers:
        n_out = int(np.ceil(OUTLIER_FRACTION * K))
        cols = rng(workload, stream + 100).permutation(K)[:n_out]
        z[:, cols] *= np.float32(OUTLIER_GAIN)
    return torch.from_numpy(z).to(dtype)


def weights_bf16(N, K, workload, stream=1):
    return normal((N, K), workload, stream, sigma=W_SIGMA, dtype=torch.bfloat16)


def block32_codes(N, K, workload, stream=1):
    """uint8 [N, K] E4M3 codes of N(0, 1) draws (torch's e4m3fn cast)."""
    z = rng(workload, stream).standard_normal(size=(N, K), dtype=np.float32)
    return torch.from_numpy(z).to(torch.float8_e4m3fn).view(torch.uint8)


def block32_scales(N, K, workload, stream=2, lo=-14, hi=7):
    """fp32 [N/32, K/32] scales 2^e with e uniform on {lo, ..., hi}."""
    e = rng(workload, stream).integers(lo, hi + 1, size=(N // 32, K // 32))
    return torch.from_numpy(np.ldexp(np.float32(1.0), e).astype(np.float32))


def e4m3_codes(rows, K, workload, stream):
    """uint8 [rows, K] codes drawn uniformly from the 254 finite E4M3 codes
    (every byte but 0x7F and 0xFF)."""
    v = rng(workload, stream).integers(0, 254, size=(rows, K), dtype=np.uint8)
    v += v >= 0x7F
    return torch.from_numpy(v)


def block_scales(rows, cols, workload, stream, lo=-10.0, hi=-4.0):
    """fp32 [rows, cols] positive scales 2^u, u uniform on [lo, hi)."""
    u = rng(workload, stream).uniform(lo, hi, size=(rows, cols))
    return torch.from_numpy(np.exp2(u).astype(np.float32))


def workload(wid, M=None):
    """Inputs of workload 0, 1 or 2 as a dict of CPU tensors."""
    if wid == 0:
        return {"x": activations(4, 512, 0), "w": weights_bf16(512, 512, 0)}
    if wid == 1:
        return {"x": activations(1 if M is None else M, 4096, 1), "w": weights_bf16(4096, 4096, 1)}
    if wid == 2:
        return {"x": activations(4096 if M is None else M, 4096, 2, outliers=True),
                "w": weights_bf16(4096, 4096, 2)}
    raise ValueError(f"workload {wid} has no single (x, w) pair")
