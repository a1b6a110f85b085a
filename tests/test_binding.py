"""The Python binding refuses, before any C call, arguments whose sizes the
C functions cannot see: wrong dtype, wrong shape for the sizes the first
operands imply, non-contiguous views, a wrong block size, and host tensors
where device memory is required (or device tensors for the host packer).
Every call here is refused by the binding, so no kernel is launched and no
GPU is needed."""

import pytest
import torch

import blockwise_scaled_fp8_amd as bfp8
from blockwise_scaled_fp8_amd import _lib

M, N, K = 4, 256, 512
U8, F32, BF, H = torch.uint8, torch.float32, torch.bfloat16, torch.float16


def t(shape, dtype):
    return torch.zeros(shape, dtype=dtype)


def good_w8a8():
    return dict(xq=t((M, K), U8), xs=t((M, K // 128), F32), wq=t((N, K), U8), ws=t((N // 128, K // 128), F32),
                y=t((M, N), BF))


def refused(fn, status, *args, **kw):
    with pytest.raises(bfp8.Bfp8Error) as e:
        fn(*args, **kw)
    assert e.value.name == status, str(e.value)
    assert e.value.detail
    return str(e.value)


@pytest.mark.parametrize("name,bad,status", [
    ("xq", t((M, K), torch.int8), "BFP8_E_DTYPE"),
    ("xq", t((M, K, 1), U8), "BFP8_E_SHAPE"),
    ("xs", t((M, K // 128 + 1), F32), "BFP8_E_SHAPE"),
    ("xs", t((M, K // 128), BF), "BFP8_E_DTYPE"),
    ("wq", t((N, K + 128), U8), "BFP8_E_SHAPE"),
    ("wq", t((K, N), U8).t(), "BFP8_E_SHAPE"),          # transposed view: not contiguous
    ("ws", t((K // 128, N // 128), F32), "BFP8_E_SHAPE"),
    ("ws", t((N // 128, K // 128), torch.float64), "BFP8_E_DTYPE"),
    ("y", t((N, M), BF), "BFP8_E_SHAPE"),
    ("y", t((M, N), torch.int16), "BFP8_E_DTYPE"),
    ("y", t((M, 2 * N), BF)[:, ::2], "BFP8_E_SHAPE"),   # strided view
    ("y", None, "BFP8_E_NULL"),
])
@pytest.mark.parametrize("fn", [bfp8.bfp8_gemm_w8a8_blk128, bfp8.bfp8_gemm_w8a8_blk128_noalloc])
def test_w8a8_refusals(name, bad, status, fn):
    a = good_w8a8()
    a[name] = bad
    refused(fn, status, a["xq"], a["xs"], a["wq"], a["ws"], a["y"])


def test_w8a8_host_tensors_refused():
    a = good_w8a8()
    msg = refused(bfp8.bfp8_gemm_w8a8_blk128, "BFP8_E_NULL", a["xq"], a["xs"], a["wq"], a["ws"], a["y"])
    assert "not on the GPU" in msg


def test_w8a8_workspace_checked():
    a = good_w8a8()
    refused(bfp8.bfp8_gemm_w8a8_blk128, "BFP8_E_DTYPE", a["xq"], a["xs"], a["wq"], a["ws"], a["y"], t(256, F32))


@pytest.mark.parametrize("fn", [bfp8.bfp8_quant_gemm_w8a8_blk128, bfp8.bfp8_gemm_w8a16_blk128])
@pytest.mark.parametrize("case", ["x dtype", "x 1-D", "wq K", "ws shape", "y shape", "host"])
def test_16bit_activation_gemms_refusals(fn, case):
    x, wq, ws, y = t((M, K), BF), t((N, K), U8), t((N // 128, K // 128), F32), t((M, N), F32)
    status = "BFP8_E_SHAPE"
    if case == "x dtype":
        x, status = t((M, K), F32), "BFP8_E_DTYPE"
    elif case == "x 1-D":
        x = t((M * K,), BF)
    elif case == "wq K":
        wq = t((N, K - 128), U8)
    elif case == "ws shape":
        ws = t((N // 128 + 1, K // 128), F32)
    elif case == "y shape":
        y = t((M + 1, N), F32)
    else:
        status = "BFP8_E_NULL"
    refused(fn, status, x, wq, ws, y)


@pytest.mark.parametrize("case", ["e8m0 shape", "e8m0 dtype", "wq K", "y dtype"])
def test_blk32_refusals(case):
    Kb = 1024
    x, wq, e8, y = t((M, Kb), H), t((N, Kb), U8), t((N // 32, Kb // 32), U8), t((M, N), H)
    status = "BFP8_E_SHAPE"
    if case == "e8m0 shape":
        e8 = t((N // 32, Kb // 128), U8)
    elif case == "e8m0 dtype":
        e8, status = t((N // 32, Kb // 32), F32), "BFP8_E_DTYPE"
    elif case == "wq K":
        wq = t((N, Kb + 32), U8)
    else:
        y, status = t((M, N), torch.int32), "BFP8_E_DTYPE"
    refused(bfp8.bfp8_gemm_w8a16_blk32_ue8m0, status, x, wq, e8, y)


@pytest.mark.parametrize("case", ["xq shape", "xs shape", "x dtype"])
def test_quantize_act_refusals(case):
    x, xq, xs = t((M, 300), BF), t((M, 300), U8), t((M, 3), F32)
    status = "BFP8_E_SHAPE"
    if case == "xq shape":
        xq = t((M, 296), U8)
    elif case == "xs shape":
        xs = t((M, 2), F32)               # ceil(300 / 128) = 3 groups
    else:
        x, status = t((M, 300), torch.float64), "BFP8_E_DTYPE"
    refused(bfp8.bfp8_quantize_act_1x128, status, x, xq, xs)


def test_quantize_weight_and_dequantize_refusals():
    refused(bfp8.bfp8_quantize_weight_128x128, "BFP8_E_SHAPE", t((200, 300), BF), t((200, 300), U8), t((1, 3), F32))
    refused(bfp8.bfp8_dequantize_weight, "BFP8_E_SHAPE", t((64, 64), U8), t((2, 2), F32), 64, t((64, 64), BF))
    refused(bfp8.bfp8_dequantize_weight, "BFP8_E_SHAPE", t((64, 96), U8), t((2, 2), F32), 32, t((64, 96), BF))
    refused(bfp8.bfp8_dequantize_weight, "BFP8_E_DTYPE", t((64, 96), U8), t((2, 3), F32), 32, t((64, 96), U8))


def test_prepare_wants_host_tensors_of_the_right_shape():
    refused(bfp8.bfp8_prepare_blk32_ue8m0, "BFP8_E_SHAPE", t((64, 64), U8), t((2, 3), F32))
    refused(bfp8.bfp8_prepare_blk32_ue8m0, "BFP8_E_DTYPE", t((64, 64), U8), t((2, 2), torch.float64))
    refused(bfp8.bfp8_prepare_blk32_ue8m0, "BFP8_E_SHAPE", t((64,), U8), t((2, 2), F32))


def test_every_entry_point_with_tensor_arguments_checks_them():
    """Each C function that takes buffers is reached only through a binding
    function that refuses bad tensors (the refusal tests above cover them)."""
    covered = {"bfp8_quantize_act_1x128", "bfp8_quantize_weight_128x128", "bfp8_dequantize_weight",
               "bfp8_gemm_w8a8_blk128", "bfp8_gemm_w8a8_blk128_noalloc", "bfp8_quant_gemm_w8a8_blk128",
               "bfp8_gemm_w8a16_blk128",
               "bfp8_gemm_w8a16_blk32_ue8m0", "bfp8_prepare_blk32_ue8m0"}
    pointer_args = {n for n, (_, args) in _lib.SIGNATURES.items() if args.count(_lib._P) >= 2}
    assert pointer_args <= covered, pointer_args - covered
