"""C-ABI tests that need no GPU: the library loads, exports every function
include/bfp8.h declares, rejects bad arguments before any HIP call, and its
host-side block-32 scale packer agrees with the oracle's validator on every
refusal class.  Every argument set below fails at least one check, so no
kernel is ever launched by this file."""

import ctypes
import os
import re
import subprocess

import numpy as np
import pytest
import torch

import blockwise_scaled_fp8_amd as bfp8
from blockwise_scaled_fp8_amd import _lib
from oracle import prepare_blk32_ue8m0, Refusal

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bfp8.h")

# Fake, 16-byte-aligned, never-dereferenced addresses.
A = 0x10000
B = 0x20000
C = 0x30000
Y = 0x40000
MISALIGNED = 0x50008


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(bfp8_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return bfp8.load()


def test_every_declared_symbol_is_exported(lib):
    names = _declared()
    assert len(names) == 14
    assert sorted(_lib.SIGNATURES) == names
    nm = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], stdout=subprocess.PIPE, text=True).stdout
    exported = set(re.findall(r" T (bfp8_\w+)", nm))
    for n in names:
        assert n in exported, n
        assert getattr(lib, n) is not None


def test_status_strings(lib):
    for code, name in _lib.STATUS_NAMES.items():
        assert bfp8.bfp8_status_string(code) != "unknown status", name
    assert bfp8.bfp8_status_string(999) == "unknown status"


def test_limits(lib):
    w8a8 = bfp8.bfp8_get_limits(bfp8.OP_GEMM_W8A8_BLK128)
    assert w8a8 == {"k_multiple": 128, "n_multiple": 16, "align_bytes": 16, "m_stream_max": 16}
    assert bfp8.bfp8_get_limits(bfp8.OP_GEMM_W8A16_BLK32_UE8M0)["n_multiple"] == 32
    assert bfp8.bfp8_get_limits(bfp8.OP_GEMM_W8A16_BLK128)["m_stream_max"] == 16
    assert lib.bfp8_get_limits(77, None, None, None, None) == 10


def test_quant_gemm_workspace_and_limits(lib):
    op = bfp8.OP_QUANT_GEMM_W8A8_BLK128
    # quantised in registers (M <= 8 where the codes call streams): the
    # streaming kernel's split-K plan only (N = 512, K = 12288: counters of 32
    # 16x16 tiles, then 8 fp32 partial tiles each, K split 8 ways)
    for M, N, K in [(1, 4096, 4096), (8, 512, 12288), (4, 512, 512), (8, 1024, 4096)]:
        assert bfp8.bfp8_workspace_bytes(op, M, N, K) == bfp8.bfp8_workspace_bytes(bfp8.OP_GEMM_W8A8_BLK128, M, N, K)
    assert bfp8.bfp8_workspace_bytes(op, 8, 512, 12288) == 256 + 32 * 8 * 256 * 4
    assert bfp8.bfp8_workspace_bytes(op, 8, 1024, 4096) == 0     # K up to 8192 is never split
    # staged codes: W8A8 workspace + M*K codes + M*K/128 scales, each 256-aligned
    r = lambda v: (v + 255) // 256 * 256
    for M, N, K in [(4096, 4096, 4096), (64, 4096, 4096), (17, 384, 640), (9, 1024, 4096), (16, 4096, 4096),
                    (8, 1024, 12288)]:
        t = bfp8.bfp8_workspace_bytes(bfp8.OP_GEMM_W8A8_BLK128, M, N, K)
        assert bfp8.bfp8_workspace_bytes(op, M, N, K) == r(t) + r(M * K) + r(4 * M * (K // 128))
    assert bfp8.bfp8_get_limits(op)["m_stream_max"] == 16


@pytest.mark.parametrize("args,expect", [
    ((0, 0, B, C, Y, 0, 4, 512, 512, None, 0, None), 1),          # null x
    ((A, 2, B, C, Y, 0, 4, 512, 512, None, 0, None), 3),          # fp32 activations
    ((A, 0, B, C, Y, 0, 4, 520, 512, None, 0, None), 2),          # N % 16
    ((A, 0, B, C, Y, 0, 4, 512, 500, None, 0, None), 2),          # K % 128
    ((A, 0, B, C, Y, 0, 64, 512, 512, None, 0, None), 5),         # codes need a workspace above M = 8
    ((A, 0, B, C, Y, 0, 12, 512, 512, None, 0, None), 5),
    ((A, 0, B, C, MISALIGNED, 0, 4, 512, 512, None, 0, None), 4),
])
def test_quant_gemm_validation(lib, args, expect):
    assert lib.bfp8_quant_gemm_w8a8_blk128(*args) == expect


def test_workspace_sizes(lib):
    # o_proj decode needs no split-K; a narrow projection does
    assert bfp8.bfp8_workspace_bytes(bfp8.OP_GEMM_W8A8_BLK128, 1, 4096, 4096) == 0
    assert bfp8.bfp8_workspace_bytes(bfp8.OP_GEMM_W8A8_BLK128, 1, 512, 12288) > 0
    assert bfp8.bfp8_workspace_bytes(bfp8.OP_GEMM_W8A8_BLK128, 1, 1024, 4096) == 0   # K not split up to 8192
    # all-token kernel with K split 4 ways: counters (64 tiles, 256-byte aligned) + 4 fp32 partial 16x16 tiles each
    assert bfp8.bfp8_workspace_bytes(bfp8.OP_GEMM_W8A8_BLK128, 1, 1024, 12288) == 256 + 64 * 4 * 256 * 4
    assert bfp8.bfp8_workspace_bytes(bfp8.OP_GEMM_W8A8_BLK128, 4096, 1024, 4096) == 0   # 128x128 tiles
    assert bfp8.bfp8_workspace_bytes(bfp8.OP_GEMM_W8A8_BLK128, 4096, 4096, 4096) == 0   # 256x256 tiles
    # 16 < M <= 32, and K <= 4096 where the launch fits one round: one
    # workgroup per 16, 32 or 64 weight rows holds every token of its group
    # over all of K, no workspace
    assert bfp8.bfp8_workspace_bytes(bfp8.OP_GEMM_W8A8_BLK128, 32, 1024, 4096) == 0
    assert bfp8.bfp8_workspace_bytes(bfp8.OP_GEMM_W8A8_BLK128, 32, 12288, 4096) == 0
    assert bfp8.bfp8_workspace_bytes(bfp8.OP_GEMM_W8A8_BLK128, 64, 4096, 4096) == 0
    assert bfp8.bfp8_workspace_bytes(bfp8.OP_GEMM_W8A8_BLK128, 64, 12288, 4096) == 0
    assert bfp8.bfp8_workspace_bytes(bfp8.OP_GEMM_W8A8_BLK128, 256, 4096, 4096) == 0
    # ... while 12288 x 4096 at M = 128 is tiled (128x128 tiles, K split 2
    # ways: 192 workgroups in one round), and so are 4096 x 12288 at M = 64
    # (128x64 tiles, K split 8 ways) and M = 256 (128x128, K split 4 ways)
    assert bfp8.bfp8_workspace_bytes(bfp8.OP_GEMM_W8A8_BLK128, 128, 12288, 4096) == 512 + 96 * 2 * 128 * 128 * 4
    assert bfp8.bfp8_workspace_bytes(bfp8.OP_GEMM_W8A8_BLK128, 64, 4096, 12288) == 256 + 32 * 8 * 128 * 64 * 4
    assert bfp8.bfp8_workspace_bytes(bfp8.OP_GEMM_W8A8_BLK128, 256, 4096, 12288) == 256 + 32 * 2 * 4 * 128 * 128 * 4
    # mid M: 64x128 tiles, K split 4 ways -> counters + 4 fp32 partial tiles per output tile
    assert bfp8.bfp8_workspace_bytes(bfp8.OP_GEMM_W8A8_BLK128, 100, 4096, 8192) == 256 + 64 * 4 * 64 * 128 * 4
    assert bfp8.bfp8_workspace_bytes(bfp8.OP_GEMM_W8A8_BLK128, 100, 4096, 4096) == 0    # all-token kernel
    assert bfp8.bfp8_workspace_bytes(bfp8.OP_GEMM_W8A8_BLK128, 64, 384, 640) == 0      # K too short to split
    assert bfp8.bfp8_workspace_bytes(bfp8.OP_QUANT_ACT_1X128, 1, 4096, 4096) == 0
    # one token with K <= 4096 runs the dot-product kernels, which need none,
    # for every blk128 GEMM and the fused call (staged codes otherwise need room)
    for op in (bfp8.OP_GEMM_W8A8_BLK128, bfp8.OP_QUANT_GEMM_W8A8_BLK128, bfp8.OP_GEMM_W8A16_BLK128):
        for n, k in ((16, 128), (1024, 4096), (12288, 4096), (2064, 3968)):
            assert bfp8.bfp8_workspace_bytes(op, 1, n, k) == 0, (op, n, k)
    # past K = 4096 one token streams, the fused call quantising in registers:
    # its workspace is the codes call's split-K workspace
    assert bfp8.bfp8_workspace_bytes(bfp8.OP_QUANT_GEMM_W8A8_BLK128, 1, 512, 12288) == \
        bfp8.bfp8_workspace_bytes(bfp8.OP_GEMM_W8A8_BLK128, 1, 512, 12288) > 0


@pytest.mark.parametrize("args,expect", [
    ((0, 0, 4, 512, A, B, None), 1),                 # null x
    ((A, 0, 4, 512, 0, B, None), 1),                 # null xq
    ((A, 0, 0, 512, B, C, None), 2),                 # M = 0
    ((A, 0, 4, 500, B, C, None), 2),                 # K % 8
    ((A, 0, 4, 4, B, C, None), 2),                   # K < 8
    ((A, 2, 4, 512, B, C, None), 3),                 # fp32 input
    ((MISALIGNED, 0, 4, 512, B, C, None), 4),        # misaligned x
])
def test_quantize_act_validation(lib, args, expect):
    assert lib.bfp8_quantize_act_1x128(*args) == expect


@pytest.mark.parametrize("args,expect", [
    ((0, 0, 512, 512, A, B, None), 1),
    ((A, 0, 512, 12, B, C, None), 2),
    ((A, 5, 512, 512, B, C, None), 3),
    ((A, 0, 512, 512, B, MISALIGNED, None), 4),
])
def test_quantize_weight_validation(lib, args, expect):
    assert lib.bfp8_quantize_weight_128x128(*args) == expect


@pytest.mark.parametrize("args,expect", [
    ((0, B, 32, C, 0, 64, 64, None), 1),             # null codes
    ((A, 0, 32, C, 0, 64, 64, None), 1),             # null scales
    ((A, B, 32, 0, 0, 64, 64, None), 1),             # null output
    ((A, B, 64, C, 0, 64, 64, None), 2),             # block other than 32 or 128
    ((A, B, 32, C, 0, 0, 64, None), 2),              # N = 0
    ((A, B, 128, C, 0, 64, 12, None), 2),            # K % 8
    ((A, B, 32, C, 7, 64, 64, None), 3),             # output dtype
    ((A, B, 32, MISALIGNED, 1, 64, 64, None), 4),    # misaligned output
])
def test_dequantize_weight_validation(lib, args, expect):
    assert lib.bfp8_dequantize_weight(*args) == expect


def _w8a8(M=4, N=512, K=512, y_dtype=0, xq=A, ws_ptr=C, y=Y, workspace=None, wbytes=0):
    return (xq, B, A, ws_ptr, y, y_dtype, M, N, K, workspace, wbytes, None)


@pytest.mark.parametrize("kw,expect", [
    (dict(xq=0), 1),
    (dict(y=0), 1),
    (dict(M=0), 2),
    (dict(N=520), 2),                                 # N % 16
    (dict(N=0), 2),
    (dict(K=500), 2),                                 # K % 128
    (dict(K=0), 2),
    (dict(y_dtype=7), 3),
    (dict(y=MISALIGNED), 4),
    (dict(M=1, N=512, K=12288), 5),                   # split-K plan needs a workspace
    (dict(M=64, N=256, K=(1 << 23) + 128), 2),        # K limit (tiled kernel)
    (dict(M=1, N=256, K=(1 << 23) + 128), 2),         # K limit (streaming kernel)
    (dict(M=100, N=1024, K=8192), 5),                 # mid-M split-K plan needs a workspace
])
def test_w8a8_validation(lib, kw, expect):
    assert lib.bfp8_gemm_w8a8_blk128(*_w8a8(**kw)) == expect


def test_w8a8_workspace_too_small(lib):
    need = bfp8.bfp8_workspace_bytes(bfp8.OP_GEMM_W8A8_BLK128, 1, 512, 12288)
    assert lib.bfp8_gemm_w8a8_blk128(*_w8a8(M=1, N=512, K=12288, workspace=A, wbytes=need - 1)) == 5
    assert lib.bfp8_gemm_w8a8_blk128(*_w8a8(M=1, N=512, K=12288, workspace=MISALIGNED, wbytes=need, y=0)) == 1


@pytest.mark.parametrize("x_dtype,y_dtype,N,expect", [
    (2, 0, 512, 3), (0, 9, 512, 3), (0, 0, 500, 2),
])
def test_w8a16_validation(lib, x_dtype, y_dtype, N, expect):
    assert lib.bfp8_gemm_w8a16_blk128(A, x_dtype, B, C, Y, y_dtype, 4, N, 512, None, 0, None) == expect


@pytest.mark.parametrize("x_dtype,N,K,expect", [
    (0, 4096, 7168, 3),          # bf16 activations are not offered for block-32
    (1, 4080, 7168, 2),          # N % 32
    (1, 4096, 7200, 2),          # K % 128
])
def test_blk32_validation(lib, x_dtype, N, K, expect):
    assert lib.bfp8_gemm_w8a16_blk32_ue8m0(A, x_dtype, B, C, Y, 1, 4, N, K, None, 0, None) == expect


# ------------------------------------------------ host packer vs oracle ----

_REFUSAL_OF_STATUS = {0: Refusal.OK, 6: Refusal.NAN_CODE, 7: Refusal.SCALE_NOT_POW2, 8: Refusal.SCALE_WINDOW}


def _both(wq, s):
    st, e8, bad = bfp8.bfp8_prepare_blk32_ue8m0(torch.from_numpy(wq), torch.from_numpy(s))
    ref_st, ref_e8, ref_bad = prepare_blk32_ue8m0(wq, s)
    assert _REFUSAL_OF_STATUS[st] is ref_st and bad == ref_bad
    if ref_e8 is not None:
        np.testing.assert_array_equal(e8.numpy(), ref_e8)
    return st


def test_prepare_accepts_full_window():
    g = np.random.default_rng(0)
    wq = g.choice([c for c in range(256) if (c & 0x7F) != 0x7F], size=(128, 256)).astype(np.uint8)
    s = np.ldexp(np.float32(1), g.integers(-14, 8, size=(4, 8))).astype(np.float32)
    assert _both(wq, s) == 0


@pytest.mark.parametrize("value", [3.0, 0.0, -1.0, -0.5, np.inf, -np.inf, np.nan, 1.5 * 2.0 ** -20,
                                   2.0 ** -15, 2.0 ** 8, 2.0 ** -130, 2.0 ** 100, 2.0 ** -14, 2.0 ** 7])
def test_prepare_scale_refusals_match_oracle(value):
    wq = np.zeros((64, 128), np.uint8)
    s = np.ones((2, 4), np.float32)
    s[1, 2] = value
    _both(wq, s)


@pytest.mark.parametrize("pos", [(0, 0), (5, 17), (63, 127)])
@pytest.mark.parametrize("code", [0x7F, 0xFF])
def test_prepare_nan_code_refusals_match_oracle(pos, code):
    wq = np.zeros((64, 128), np.uint8)
    wq[pos] = code
    s = np.full((2, 4), 3.0, np.float32)      # bad scales too: the codes are reported first
    assert _both(wq, s) == 6


def test_prepare_validation(lib):
    bad = ctypes.c_int64(5)
    assert lib.bfp8_prepare_blk32_ue8m0(None, None, 32, 32, None, ctypes.byref(bad)) == 1
    assert bad.value == -1
    buf = (ctypes.c_uint8 * 16384)()
    assert lib.bfp8_prepare_blk32_ue8m0(buf, buf, 48, 128, buf, ctypes.byref(bad)) == 2
    # K must be whole 128-K blocks, the unit the block-32 GEMM streams, so that
    # a layer the packer accepts is one the GEMM accepts
    assert lib.bfp8_prepare_blk32_ue8m0(buf, buf, 64, 96, buf, ctypes.byref(bad)) == 2
    assert lib.bfp8_gemm_w8a16_blk32_ue8m0(A, 1, B, C, Y, 1, 4, 64, 96, None, 0, None) == 2
    k_mult = ctypes.c_int64(0)
    assert lib.bfp8_get_limits(bfp8.OP_GEMM_W8A16_BLK32_UE8M0, ctypes.byref(k_mult), None, None, None) == 0
    assert k_mult.value == 128


# --------------------------------------------------------------- build ----

def test_kernels_have_no_scratch_and_no_spills():
    from blockwise_scaled_fp8_amd.build import kernel_resources
    res = kernel_resources()
    assert len(res) >= 7
    for name, r in res.items():
        assert r["ScratchSize [bytes/lane]"] == 0, name
        assert r["VGPRs Spill"] == 0 and r["SGPRs Spill"] == 0, name
        assert r["LDS Size [bytes/block]"] <= 160 * 1024, name


# ------------------------------------------------ allocation-free W8A8 ----

def test_noalloc_scratch_size_matches_the_header():
    text = open(HEADER).read()
    assert "#define BFP8_NOALLOC_SCRATCH_BYTES ((size_t)(16u << 20) + 4096u)" in text
    assert bfp8.NOALLOC_SCRATCH_BYTES == (16 << 20) + 4096


def test_noalloc_scratch_covers_every_planned_workspace():
    """The planners keep every W8A8 workspace within the static scratch, so
    the allocation-free call serves every shape the workspace call does."""
    import itertools
    worst = 0
    for M, N, K in itertools.product(list(range(1, 70)) + [96, 128, 129, 200, 256, 300, 400, 512, 768, 1000, 1024,
                                                           2048, 4096, 8192],
                                     [16, 64, 256, 512, 1024, 2048, 4096, 8192, 12288, 16384, 65536],
                                     [128, 512, 1024, 2048, 4096, 8192, 12288, 16384, 65536]):
        worst = max(worst, bfp8.bfp8_workspace_bytes(bfp8.OP_GEMM_W8A8_BLK128, M, N, K))
    assert 0 < worst <= bfp8.NOALLOC_SCRATCH_BYTES


@pytest.mark.parametrize("args,expect", [
    (dict(xq=0), 1), (dict(y=0), 1), (dict(M=0), 2), (dict(N=24), 2), (dict(K=200), 2), (dict(y_dtype=7), 3),
    (dict(y=MISALIGNED), 4), (dict(xs=MISALIGNED), 4),
])
def test_noalloc_validation(lib, args, expect):
    a = dict(xq=A, xs=B, wq=C, ws=B, y=Y, y_dtype=0, M=4, N=256, K=512)
    a.update(args)
    assert lib.bfp8_gemm_w8a8_blk128_noalloc(a["xq"], a["xs"], a["wq"], a["ws"], a["y"], a["y_dtype"], a["M"],
                                            a["N"], a["K"], None) == expect
