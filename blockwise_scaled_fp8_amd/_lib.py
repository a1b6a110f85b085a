"""ctypes binding of libbfp8.so — argument marshalling only.

Each function has the name of the C entry point it calls and takes torch
tensors where the C function takes device pointers; every step of the
computation runs in the library's HIP kernels.  Work is enqueued on the
current torch stream.  A missing library raises at load time; a nonzero
status raises Bfp8Error with the library's status text.  There is no
fallback of any kind.

The C functions take bare pointers and cannot see buffer sizes, so before
each call the binding checks what only it can: every tensor lives on the
current GPU (host tensors for the host-only packer), is contiguous, has the
dtype the C argument expects, and has the shape that M, N and K (taken from
the first operands) imply.  A mismatch raises Bfp8Error before anything is
enqueued.  Arithmetic and kernel choice stay in the library.
"""

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libbfp8.so")

# Values of the C enums and constants in include/bfp8.h.
NOALLOC_SCRATCH_BYTES = (16 << 20) + 4096
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
    "bfp8_gemm_w8a8_blk128_noalloc": (_I, [_P, _P, _P, _P, _P, _I, _I64, _I64, _I64, _P]),
    "bfp8_quant_gemm_w8a8_blk128": (_I, [_P, _I, _P, _P, _P, _I, _I64, _I64, _I64, _P, _SZ, _P]),
    "bfp8_gemm_w8a16_blk128": (_I, [_P, _I, _P, _P, _P, _I, _I64, _I64, _I64, _P, _SZ, _P]),
    "bfp8_gemm_w8a16_blk32_ue8m0": (_I, [_P, _I, _P, _P, _P, _I, _I64, _I64, _I64, _P, _SZ, _P]),
    "bfp8_prepare_blk32_ue8m0": (_I, [_P, _P, _I64, _I64, _P, ctypes.POINTER(_I64)]),
    "bfp8_workspace_bytes": (_SZ, [_I, _I64, _I64, _I64]),
    "bfp8_get_limits": (_I, [_I] + [ctypes.POINTER(_I64)] * 4),
    "bfp8_get_plan": (_I, [_I, _I64, _I64, _I64, _P]),
    "bfp8_kernel_name": (ctypes.c_char_p, [_I]),
    "bfp8_status_string": (ctypes.c_char_p, [_I]),
}


class Plan(ctypes.Structure):
    """struct bfp8_plan of include/bfp8.h."""
    _fields_ = [("kernel", ctypes.c_int32), ("quant_kernel", ctypes.c_int32), ("tile_n", ctypes.c_int32),
                ("tile_m", ctypes.c_int32), ("waves", ctypes.c_int32), ("splits", ctypes.c_int32),
                ("workgroups", ctypes.c_int64), ("workspace_bytes", ctypes.c_uint64)]

_lib = None


class Bfp8Error(RuntimeError):
    """A nonzero status from the library, or an argument the binding refused
    before calling it (then `detail` says which and why)."""

    def __init__(self, status, where, detail=None):
        self.status = status
        self.name = STATUS_NAMES.get(status, str(status))
        self.detail = detail
        text = detail if detail is not None else load().bfp8_status_string(status).decode()
        super().__init__(f"{where}: {self.name}: {text}")


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


_E_NULL, _E_SHAPE, _E_DTYPE = 1, 2, 3
_U8, _F32 = (torch.uint8,), (torch.float32,)
_X16 = (torch.bfloat16, torch.float16)
_OUT = (torch.bfloat16, torch.float16, torch.float32)


def _cdiv(a, b):
    return -(-a // b)


def _arg(where, name, t, dtypes, shape=None, ndim=None):
    """Refuse a tensor argument that the C call cannot take: missing, of the
    wrong dtype, not contiguous, or of a shape other than the one the call's
    sizes imply.  Where it lives is checked afterwards by _placed, once every
    argument has passed these checks."""
    if t is None:
        raise Bfp8Error(_E_NULL, where, f"{name} is None")
    if not isinstance(t, torch.Tensor):
        raise Bfp8Error(_E_NULL, where, f"{name} is not a torch tensor")
    if t.dtype not in dtypes:
        raise Bfp8Error(_E_DTYPE, where, f"{name} has dtype {t.dtype}, expected one of {list(dtypes)}")
    if ndim is not None and t.dim() != ndim:
        raise Bfp8Error(_E_SHAPE, where, f"{name} must be {ndim}-D, got shape {tuple(t.shape)}")
    if not t.is_contiguous():
        raise Bfp8Error(_E_SHAPE, where, f"{name} is not contiguous (strides {t.stride()})")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise Bfp8Error(_E_SHAPE, where, f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _placed(where, device=True, **tensors):
    """Every tensor on the current GPU (device=True) or in host memory."""
    for name, t in tensors.items():
        if t is None:
            continue
        if device:
            if not t.is_cuda:
                raise Bfp8Error(_E_NULL, where, f"{name} is on {t.device}, not on the GPU")
            if t.device.index != torch.cuda.current_device():
                raise Bfp8Error(_E_NULL, where, f"{name} is on {t.device}, the current device is "
                                                f"cuda:{torch.cuda.current_device()}")
        elif t.device.type != "cpu":
            raise Bfp8Error(_E_NULL, where, f"{name} must be a host tensor, got {t.device}")


def _mat(where, name, t, dtypes):
    """A 2-D operand whose shape defines sizes; returns its (rows, cols)."""
    _arg(where, name, t, dtypes, ndim=2)
    return t.shape


def _workspace_arg(where, workspace):
    if workspace is not None:
        _arg(where, "workspace", workspace, _U8)


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _check(status, where):
    if status != 0:
        raise Bfp8Error(status, where)


def _ws(workspace):
    return (None, 0) if workspace is None else (_ptr(workspace), workspace.numel() * workspace.element_size())


def bfp8_quantize_act_1x128(x, xq, xs):
    w = "bfp8_quantize_act_1x128"
    M, K = _mat(w, "x", x, _X16)
    _arg(w, "xq", xq, _U8, (M, K))
    _arg(w, "xs", xs, _F32, (M, _cdiv(K, 128)))
    _placed(w, x=x, xq=xq, xs=xs)
    _check(load().bfp8_quantize_act_1x128(_ptr(x), _dtype_code(x), M, K, _ptr(xq), _ptr(xs), _stream()), w)


def bfp8_quantize_weight_128x128(w_, wq, ws):
    w = "bfp8_quantize_weight_128x128"
    N, K = _mat(w, "w", w_, _X16)
    _arg(w, "wq", wq, _U8, (N, K))
    _arg(w, "ws", ws, _F32, (_cdiv(N, 128), _cdiv(K, 128)))
    _placed(w, w=w_, wq=wq, ws=ws)
    _check(load().bfp8_quantize_weight_128x128(_ptr(w_), _dtype_code(w_), N, K, _ptr(wq), _ptr(ws), _stream()), w)


def bfp8_dequantize_weight(wq, scales, block, w_):
    w = "bfp8_dequantize_weight"
    N, K = _mat(w, "wq", wq, _U8)
    if block not in (32, 128):
        raise Bfp8Error(_E_SHAPE, w, f"block must be 32 or 128, got {block}")
    _arg(w, "scales", scales, _F32, (_cdiv(N, block), _cdiv(K, block)))
    _arg(w, "w", w_, _OUT, (N, K))
    _placed(w, wq=wq, scales=scales, w=w_)
    _check(load().bfp8_dequantize_weight(_ptr(wq), _ptr(scales), block, _ptr(w_), _dtype_code(w_), N, K, _stream()),
           w)


def _weights_blk128(w, wq, ws, K):
    N, Kw = _mat(w, "wq", wq, _U8)
    if Kw != K:
        raise Bfp8Error(_E_SHAPE, w, f"wq has K = {Kw}, the activations have K = {K}")
    _arg(w, "ws", ws, _F32, (_cdiv(N, 128), _cdiv(K, 128)))
    return N


def bfp8_gemm_w8a8_blk128(xq, xs, wq, ws, y, workspace=None):
    w = "bfp8_gemm_w8a8_blk128"
    M, K = _mat(w, "xq", xq, _U8)
    _arg(w, "xs", xs, _F32, (M, _cdiv(K, 128)))
    N = _weights_blk128(w, wq, ws, K)
    _arg(w, "y", y, _OUT, (M, N))
    _workspace_arg(w, workspace)
    _placed(w, xq=xq, xs=xs, wq=wq, ws=ws, y=y, workspace=workspace)
    wsp, wsb = _ws(workspace)
    _check(load().bfp8_gemm_w8a8_blk128(_ptr(xq), _ptr(xs), _ptr(wq), _ptr(ws), _ptr(y), _dtype_code(y),
                                        M, N, K, wsp, wsb, _stream()), w)


def bfp8_gemm_w8a8_blk128_noalloc(xq, xs, wq, ws, y):
    """bfp8_gemm_w8a8_blk128 with the library's own per-GPU scratch as the
    workspace (for callers that cannot allocate; calls on one GPU must not
    overlap in time)."""
    w = "bfp8_gemm_w8a8_blk128_noalloc"
    M, K = _mat(w, "xq", xq, _U8)
    _arg(w, "xs", xs, _F32, (M, _cdiv(K, 128)))
    N = _weights_blk128(w, wq, ws, K)
    _arg(w, "y", y, _OUT, (M, N))
    _placed(w, xq=xq, xs=xs, wq=wq, ws=ws, y=y)
    _check(load().bfp8_gemm_w8a8_blk128_noalloc(_ptr(xq), _ptr(xs), _ptr(wq), _ptr(ws), _ptr(y), _dtype_code(y),
                                                M, N, K, _stream()), w)


def bfp8_quant_gemm_w8a8_blk128(x, wq, ws, y, workspace=None):
    w = "bfp8_quant_gemm_w8a8_blk128"
    M, K = _mat(w, "x", x, _X16)
    N = _weights_blk128(w, wq, ws, K)
    _arg(w, "y", y, _OUT, (M, N))
    _workspace_arg(w, workspace)
    _placed(w, x=x, wq=wq, ws=ws, y=y, workspace=workspace)
    wsp, wsb = _ws(workspace)
    _check(load().bfp8_quant_gemm_w8a8_blk128(_ptr(x), _dtype_code(x), _ptr(wq), _ptr(ws), _ptr(y),
                                              _dtype_code(y), M, N, K, wsp, wsb, _stream()), w)


def bfp8_gemm_w8a16_blk128(x, wq, ws, y, workspace=None):
    w = "bfp8_gemm_w8a16_blk128"
    M, K = _mat(w, "x", x, _X16)
    N = _weights_blk128(w, wq, ws, K)
    _arg(w, "y", y, _OUT, (M, N))
    _workspace_arg(w, workspace)
    _placed(w, x=x, wq=wq, ws=ws, y=y, workspace=workspace)
    wsp, wsb = _ws(workspace)
    _check(load().bfp8_gemm_w8a16_blk128(_ptr(x), _dtype_code(x), _ptr(wq), _ptr(ws), _ptr(y), _dtype_code(y),
                                         M, N, K, wsp, wsb, _stream()), w)


def bfp8_gemm_w8a16_blk32_ue8m0(x, wq, e8m0, y, workspace=None):
    w = "bfp8_gemm_w8a16_blk32_ue8m0"
    M, K = _mat(w, "x", x, _X16)
    N, Kw = _mat(w, "wq", wq, _U8)
    if Kw != K:
        raise Bfp8Error(_E_SHAPE, w, f"wq has K = {Kw}, the activations have K = {K}")
    _arg(w, "e8m0", e8m0, _U8, (_cdiv(N, 32), _cdiv(K, 32)))
    _arg(w, "y", y, _OUT, (M, N))
    _workspace_arg(w, workspace)
    _placed(w, x=x, wq=wq, e8m0=e8m0, y=y, workspace=workspace)
    wsp, wsb = _ws(workspace)
    _check(load().bfp8_gemm_w8a16_blk32_ue8m0(_ptr(x), _dtype_code(x), _ptr(wq), _ptr(e8m0), _ptr(y),
                                              _dtype_code(y), M, N, K, wsp, wsb, _stream()), w)


def bfp8_prepare_blk32_ue8m0(wq_host, scale_host):
    """Host tensors in, (status, e8m0 uint8 host tensor or None, bad_index) out;
    refusals are returned, not raised, so callers can act on the index."""
    w = "bfp8_prepare_blk32_ue8m0"
    wq_host = wq_host.contiguous()
    scale_host = scale_host.contiguous()
    _arg(w, "wq_host", wq_host, _U8, ndim=2)
    N, K = wq_host.shape
    _arg(w, "scale_host", scale_host, _F32, (_cdiv(N, 32), _cdiv(K, 32)))
    _placed(w, device=False, wq_host=wq_host, scale_host=scale_host)
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


def bfp8_get_plan(op, M, N, K):
    """The launch plan the library uses for op at M x N x K, as a dict with
    the kernel's name (host only, no GPU needed)."""
    p = Plan()
    _check(load().bfp8_get_plan(op, M, N, K, ctypes.byref(p)), "bfp8_get_plan")
    out = {f: getattr(p, f) for f, _ in Plan._fields_}
    out["kernel_name"] = bfp8_kernel_name(p.kernel)
    out["quant_kernel_name"] = bfp8_kernel_name(p.quant_kernel)
    return out


def bfp8_kernel_name(kernel):
    return load().bfp8_kernel_name(kernel).decode()


def bfp8_status_string(status):
    return load().bfp8_status_string(status).decode()
