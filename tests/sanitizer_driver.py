"""Host-side paths of a host-sanitized build of the library (path in argv[1]),
run by tests/test_host_sanitizer.py in a process that preloads the
AddressSanitizer runtime.  Plain ctypes and host memory only: nothing here
launches a kernel or needs a GPU.  Exits 0 when every call returns what the
header promises; a sanitizer report aborts the process instead.

Covered: the block-32 packer on success and on every refusal class (and its
reported index), the argument checks of every entry point that refuse before
any launch (NULL, shape, dtype, alignment, workspace), the plan and workspace
queries over a sweep of shapes for every op, the limits, and the names of
every status and kernel id.
"""

import ctypes
import itertools
import sys

OK, E_NULL, E_SHAPE, E_DTYPE, E_ALIGN, E_WORKSPACE, E_NAN, E_POW2, E_WINDOW, E_LAUNCH, E_OP = range(11)
OPS = range(6)
BF16, F16, F32 = 0, 1, 2


class Plan(ctypes.Structure):
    """struct bfp8_plan of include/bfp8.h."""
    _fields_ = [("kernel", ctypes.c_int32), ("quant_kernel", ctypes.c_int32), ("tile_n", ctypes.c_int32),
                ("tile_m", ctypes.c_int32), ("waves", ctypes.c_int32), ("splits", ctypes.c_int32),
                ("workgroups", ctypes.c_int64), ("workspace_bytes", ctypes.c_uint64)]


def host_array(libc, ctype, values):
    """An array of exactly len(values) elements in its own libc allocation,
    which the preloaded AddressSanitizer runtime surrounds with redzones (a
    ctypes array of Python's own would sit inside a larger arena)."""
    n = len(values)
    arr = (ctype * n).from_address(libc.malloc(n * ctypes.sizeof(ctype)))
    arr[:] = values
    return arr


def expect(got, want, what):
    if got != want:
        raise SystemExit(f"{what}: status {got}, expected {want}")


def main(path):
    lib = ctypes.CDLL(path)
    i64, vp, sz = ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t
    libc = ctypes.CDLL(None)
    libc.malloc.restype, libc.malloc.argtypes = vp, [sz]
    lib.bfp8_prepare_blk32_ue8m0.argtypes = [vp, vp, i64, i64, vp, ctypes.POINTER(i64)]
    lib.bfp8_workspace_bytes.restype = sz
    lib.bfp8_workspace_bytes.argtypes = [ctypes.c_int, i64, i64, i64]
    lib.bfp8_get_plan.argtypes = [ctypes.c_int, i64, i64, i64, ctypes.POINTER(Plan)]
    lib.bfp8_get_limits.argtypes = [ctypes.c_int] + [ctypes.POINTER(i64)] * 4
    lib.bfp8_kernel_name.restype = ctypes.c_char_p
    lib.bfp8_status_string.restype = ctypes.c_char_p
    gemm_args = [vp, vp, vp, vp, vp, ctypes.c_int, i64, i64, i64, vp, sz, vp]
    lib.bfp8_gemm_w8a8_blk128.argtypes = gemm_args
    lib.bfp8_gemm_w8a8_blk128_noalloc.argtypes = [vp, vp, vp, vp, vp, ctypes.c_int, i64, i64, i64, vp]
    gemm16_args = [vp, ctypes.c_int, vp, vp, vp, ctypes.c_int, i64, i64, i64, vp, sz, vp]
    lib.bfp8_quant_gemm_w8a8_blk128.argtypes = gemm16_args
    lib.bfp8_gemm_w8a16_blk128.argtypes = gemm16_args
    lib.bfp8_gemm_w8a16_blk32_ue8m0.argtypes = gemm16_args
    lib.bfp8_quantize_act_1x128.argtypes = [vp, ctypes.c_int, i64, i64, vp, vp, vp]
    lib.bfp8_quantize_weight_128x128.argtypes = [vp, ctypes.c_int, i64, i64, vp, vp, vp]
    lib.bfp8_dequantize_weight.argtypes = [vp, vp, i64, vp, ctypes.c_int, i64, i64, vp]

    # --- block-32 packer (host memory) -----------------------------------
    N, K = 64, 256
    wq = host_array(libc, ctypes.c_uint8, [0x38] * (N * K))           # E4M3 1.0 everywhere
    nsc = (N // 32) * (K // 32)
    scales = host_array(libc, ctypes.c_float, [2.0 ** ((i % 22) - 14) for i in range(nsc)])
    e8 = host_array(libc, ctypes.c_uint8, [0] * nsc)
    bad = i64.from_address(ctypes.addressof(host_array(libc, i64, [7])))
    expect(lib.bfp8_prepare_blk32_ue8m0(wq, scales, N, K, e8, ctypes.byref(bad)), OK, "prepare ok")
    assert bad.value == -1 and list(e8) == [((i % 22) - 14) + 127 for i in range(nsc)], (bad.value, list(e8))
    wq[N * K - 1] = 0xFF                                               # a NaN code, the last weight
    expect(lib.bfp8_prepare_blk32_ue8m0(wq, scales, N, K, e8, ctypes.byref(bad)), E_NAN, "prepare NaN code")
    assert bad.value == N * K - 1, bad.value
    wq[N * K - 1] = 0x38
    for v, st in ((3.0, E_POW2), (0.0, E_POW2), (-2.0, E_POW2), (float("inf"), E_POW2), (float("nan"), E_POW2),
                  (2.0 ** 8, E_WINDOW), (2.0 ** -15, E_WINDOW)):
        keep = scales[nsc - 1]
        scales[nsc - 1] = v
        expect(lib.bfp8_prepare_blk32_ue8m0(wq, scales, N, K, e8, ctypes.byref(bad)), st, f"prepare scale {v}")
        assert bad.value == nsc - 1, (v, bad.value)
        scales[nsc - 1] = keep
    for n, k in ((48, 256), (64, 192), (0, 256), (64, 0), (-32, 256)):
        expect(lib.bfp8_prepare_blk32_ue8m0(wq, scales, n, k, e8, ctypes.byref(bad)), E_SHAPE, f"prepare {n}x{k}")
    expect(lib.bfp8_prepare_blk32_ue8m0(None, scales, N, K, e8, ctypes.byref(bad)), E_NULL, "prepare null wq")
    expect(lib.bfp8_prepare_blk32_ue8m0(wq, scales, N, K, None, ctypes.byref(bad)), E_NULL, "prepare null out")

    # --- refusals before any launch (fake device pointers, never read) ----
    a, b = 0x10000, 0x20001            # aligned / misaligned stand-ins
    ws_small = 16
    calls = [
        ("w8a8 null", lib.bfp8_gemm_w8a8_blk128, (None, a, a, a, a, BF16, 4, 512, 512, None, 0, None), E_NULL),
        ("w8a8 M=0", lib.bfp8_gemm_w8a8_blk128, (a, a, a, a, a, BF16, 0, 512, 512, None, 0, None), E_SHAPE),
        ("w8a8 N%16", lib.bfp8_gemm_w8a8_blk128, (a, a, a, a, a, BF16, 4, 520, 512, None, 0, None), E_SHAPE),
        ("w8a8 K%128", lib.bfp8_gemm_w8a8_blk128, (a, a, a, a, a, BF16, 4, 512, 500, None, 0, None), E_SHAPE),
        ("w8a8 dtype", lib.bfp8_gemm_w8a8_blk128, (a, a, a, a, a, 7, 4, 512, 512, None, 0, None), E_DTYPE),
        ("w8a8 align", lib.bfp8_gemm_w8a8_blk128, (b, a, a, a, a, BF16, 4, 512, 512, None, 0, None), E_ALIGN),
        ("w8a8 workspace", lib.bfp8_gemm_w8a8_blk128, (a, a, a, a, a, F32, 16, 512, 12288, a, ws_small, None),
         E_WORKSPACE),
        ("noalloc null", lib.bfp8_gemm_w8a8_blk128_noalloc, (a, None, a, a, a, BF16, 4, 512, 512, None), E_NULL),
        ("noalloc shape", lib.bfp8_gemm_w8a8_blk128_noalloc, (a, a, a, a, a, BF16, 4, 512, 100, None), E_SHAPE),
        ("fused dtype", lib.bfp8_quant_gemm_w8a8_blk128, (a, F32, a, a, a, BF16, 4, 512, 512, None, 0, None),
         E_DTYPE),
        ("fused align", lib.bfp8_quant_gemm_w8a8_blk128, (a, BF16, a, b, a, BF16, 4, 512, 512, None, 0, None),
         E_ALIGN),
        ("w8a16 null", lib.bfp8_gemm_w8a16_blk128, (a, BF16, None, a, a, BF16, 4, 512, 512, None, 0, None), E_NULL),
        ("w8a16 shape", lib.bfp8_gemm_w8a16_blk128, (a, BF16, a, a, a, BF16, 4, 512, 0, None, 0, None), E_SHAPE),
        ("blk32 bf16 x", lib.bfp8_gemm_w8a16_blk32_ue8m0, (a, BF16, a, a, a, F16, 4, 512, 512, None, 0, None),
         E_DTYPE),
        ("blk32 K%128", lib.bfp8_gemm_w8a16_blk32_ue8m0, (a, F16, a, a, a, F16, 4, 512, 480, None, 0, None),
         E_SHAPE),
        ("quant act dtype", lib.bfp8_quantize_act_1x128, (a, F32, 4, 512, a, a, None), E_DTYPE),
        ("quant act null", lib.bfp8_quantize_act_1x128, (a, BF16, 4, 512, None, a, None), E_NULL),
        ("quant weight shape", lib.bfp8_quantize_weight_128x128, (a, BF16, 512, 100, a, a, None), E_SHAPE),
        ("dequant block", lib.bfp8_dequantize_weight, (a, a, 64, a, BF16, 512, 512, None), E_SHAPE),
        ("dequant align", lib.bfp8_dequantize_weight, (a, b, 128, a, BF16, 512, 512, None), E_ALIGN),
    ]
    for what, fn, args, want in calls:
        expect(fn(*args), want, what)

    # --- plans, workspaces, limits, names ---------------------------------
    ms = [0, 1, 2, 5, 8, 9, 16, 17, 32, 33, 64, 100, 128, 256, 300, 512, 1000, 4096, 8192]
    ns = [0, 16, 32, 48, 64, 384, 1024, 1040, 2064, 4096, 4112, 12288, 32768]
    ks = [0, 128, 256, 640, 1024, 2176, 4096, 7168, 8192, 12288, 12416, 16384, 1 << 20]
    plans = 0
    for op, M, N, K in itertools.product(OPS, ms, ns, ks):
        lib.bfp8_workspace_bytes(op, M, N, K)
        p = Plan()
        st = lib.bfp8_get_plan(op, M, N, K, ctypes.byref(p))
        if st == OK:
            plans += 1
            assert p.workgroups >= 0 and p.splits >= 1, (op, M, N, K)
        else:
            assert st in (E_SHAPE,), (op, M, N, K, st)
    assert plans > 1000, plans
    expect(lib.bfp8_get_plan(99, 1, 16, 128, ctypes.byref(Plan())), E_OP, "plan op")
    expect(lib.bfp8_get_plan(2, 1, 16, 128, None), E_NULL, "plan null")
    for op in OPS:
        vals = [i64() for _ in range(4)]
        expect(lib.bfp8_get_limits(op, *[ctypes.byref(v) for v in vals]), OK, f"limits {op}")
        lib.bfp8_get_limits(op, None, None, None, None)
    for k in range(-1, 40):
        assert lib.bfp8_kernel_name(k)
    for s in range(-1, 15):
        assert lib.bfp8_status_string(s)
    print("host paths ok:", plans, "plans")


if __name__ == "__main__":
    main(sys.argv[1])
