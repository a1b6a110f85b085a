"""ctypes binding of libbfp8.so — argument marshalling only.

Each function has the name of the C entry point it calls and takes torch
tensors where the C function takes device pointers; every step of the
computation runs in the library's HIP kernels.  Work is enqueued on the
current torch stream.  A missing library raises at load time; a nonzero
status raises Bfp8Error with the library's status text.  There is no
fallback of any kind.
"""

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libbfp8.so")

# Values of the C enums in include/bfp8.h.
BFP8_BF16, BFP8_F16, BFP8_F32 = 0, 1, 2
OP_QUANT_ACT_1X128 = 0
OP_QUANT_WEIGHT_128X128 = 1
OP_GEMM_W8A8_BLK128 = 2
OP_GEMM_W8A16_BLK128 = 3
OP_GEMM_W8A16_BLK32_UE8M0 = 4
OP_QUANT_GEMM_W8A8_BLK128 = 5
STATUS_NAMES = {
    0: "BFP8_OK", 1: "BFP8_E_NULL", 2: "BFP8_E_SHAPE", 3: "BFP8_E_DTYPE", 4: "BFP8_E_ALIGN",
    5: "BFP8_E_WORKSPACE", 6: "BFP8_E_NAN_CODE", 7: "BFP8_E_SCALE_NOT_POW2", 8: "BFP8_E_SCALE_WINDOW",
    9: "BFP8_E_LAUNCH", 10: "BFP8_E_OP",
}

# Every function the header declares, with its ctypes signature.
_P, _I, _I64, _SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
SIGNATURES = {
    "bfp8_quantize_act_1x128": (_I, [_P, _I, _I64, _I64, _P, _P, _P]),
    "bfp8_quantize_weight_128x128": (_I, [_P, _I, _I64, _I64, _P, _P, _P]),
    "bfp8_dequantize_weight": (_I, [_P, _P, _I64, _P, _I, _I64, _I64, _P]),
    "bfp8_gemm_w8a8_blk128": (_I, [_P, _P, _P, _P, _P, _I, _I64, _I64, _I64, _P, _SZ, _P]),
    "bfp8_quant_gemm_w8a8_blk128": (_I, [_P, _I, _P, _P, _P, _I, _I64, _I64, _I64, _P, _SZ, _P]),
    "bfp8_gemm_w8a16_blk128": (_I, [_P, _I, _P, _P, _P, _I, _I64, _I64, _I64, _P, _SZ, _P]),
    "bfp8_gemm_w8a16_blk32_ue8m0": (_I, [_P, _I, _P, _P, _P, _I, _I64, _I64, _I64, _P, _SZ, _P]),
    "bfp8_prepare_blk32_ue8m0": (_I, [_P, _P, _I64, _I64, _P, ctypes.POINTER(_I64)]),
    "bfp8_workspace_bytes": (_SZ, [_I, _I64, _I64, _I64]),
    "bfp8_get_limits": (_I, [_I] + [ctypes.POINTER(_I64)] * 4),
    "bfp8_status_string": (ctypes.c_char_p, [_I]),
}

_lib = None


class Bfp8Error(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        self.name = STATUS_NAMES.get(status, str(status))
        super().__init__(f"{where}: {self.name}: {load().bfp8_status_string(status).decode()}")


def load():
    """Load libbfp8.so (once).  Raises OSError when it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise OSError(f"{LIB_PATH} is missing: build it with blockwise_scaled_fp8_amd.build.build()")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype, fn.argtypes = res, args
        _lib = lib
    return _lib


def _dtype_code(t):
    try:
        return {torch.bfloat16: BFP8_BF16, torch.float16: BFP8_F16, torch.float32: BFP8_F32}[t.dtype]
    except KeyError:
        return -1


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _check(status, where):
    if status != 0:
        raise Bfp8Error(status, where)


def _ws(workspace):
    return (None, 0) if workspace is None else (_ptr(workspace), workspace.numel() * workspace.element_size())


def bfp8_quantize_act_1x128(x, xq, xs):
    M, K = x.shape
    _check(load().bfp8_quantize_act_1x128(_ptr(x), _dtype_code(x), M, K, _ptr(xq), _ptr(xs), _stream()),
           "bfp8_quantize_act_1x128")


def bfp8_quantize_weight_128x128(w, wq, ws):
    N, K = w.shape
    _check(load().bfp8_quantize_weight_128x128(_ptr(w), _dtype_code(w), N, K, _ptr(wq), _ptr(ws), _stream()),
           "bfp8_quantize_weight_128x128")


def bfp8_dequantize_weight(wq, scales, block, w):
    N, K = wq.shape
    _check(load().bfp8_dequantize_weight(_ptr(wq), _ptr(scales), block, _ptr(w), _dtype_code(w), N, K, _stream()),
           "bfp8_dequantize_weight")


def bfp8_gemm_w8a8_blk128(xq, xs, wq, ws, y, workspace=None):
    M, K = xq.shape
    N = wq.shape[0]
    wsp, wsb = _ws(workspace)
    _check(load().bfp8_gemm_w8a8_blk128(_ptr(xq), _ptr(xs), _ptr(wq), _ptr(ws), _ptr(y), _dtype_code(y),
                                        M, N, K, wsp, wsb, _stream()), "bfp8_gemm_w8a8_blk128")


def bfp8_quant_gemm_w8a8_blk128(x, wq, ws, y, workspace=None):
    M, K = x.shape
    N = wq.shape[0]
    wsp, wsb = _ws(workspace)
    _check(load().bfp8_quant_gemm_w8a8_blk128(_ptr(x), _dtype_code(x), _ptr(wq), _ptr(ws), _ptr(y),
                                              _dtype_code(y), M, N, K, wsp, wsb, _stream()),
           "bfp8_quant_gemm_w8a8_blk128")


def bfp8_gemm_w8a16_blk128(x, wq, ws, y, workspace=None):
    M, K = x.shape
    N = wq.shape[0]
    wsp, wsb = _ws(workspace)
    _check(load().bfp8_gemm_w8a16_blk128(_ptr(x), _dtype_code(x), _ptr(wq), _ptr(ws), _ptr(y), _dtype_code(y),
                                         M, N, K, wsp, wsb, _stream()), "bfp8_gemm_w8a16_blk128")


def bfp8_gemm_w8a16_blk32_ue8m0(x, wq, e8m0, y, workspace=None):
    M, K = x.shape
    N = wq.shape[0]
    wsp, wsb = _ws(workspace)
    _check(load().bfp8_gemm_w8a16_blk32_ue8m0(_ptr(x), _dtype_code(x), _ptr(wq), _ptr(e8m0), _ptr(y),
                                              _dtype_code(y), M, N, K, wsp, wsb, _stream()),
           "bfp8_gemm_w8a16_blk32_ue8m0")


def bfp8_prepare_blk32_ue8m0(wq_host, scale_host):
    """Host tensors in, (status, e8m0 uint8 host tensor or None, bad_index) out;
    refusals are returned, not raised, so callers can act on the index."""
    wq_host = wq_host.contiguous()
    scale_host = scale_host.contiguous()
    N, K = wq_host.shape
    out = torch.empty((N // 32, K // 32), dtype=torch.uint8)
    bad = ctypes.c_int64(-1)
    st = load().bfp8_prepare_blk32_ue8m0(_ptr(wq_host), _ptr(scale_host), N, K, _ptr(out), ctypes.byref(bad))
    return st, (out if st == 0 else None), bad.value


def bfp8_workspace_bytes(op, M, N, K):
    return int(load().bfp8_workspace_bytes(op, M, N, K))


def bfp8_get_limits(op):
    vals = [ctypes.c_int64(0) for _ in range(4)]
    _check(load().bfp8_get_limits(op, *[ctypes.byref(v) for v in vals]), "bfp8_get_limits")
    return {"k_multiple": vals[0].value, "n_multiple": vals[1].value,
            "align_bytes": vals[2].value, "m_stream_max": vals[3].value}


def bfp8_status_string(status):
    return load().bfp8_status_string(status).decode()
