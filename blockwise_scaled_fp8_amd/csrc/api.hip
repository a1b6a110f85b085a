// C entry points of libbfp8: argument validation (before any HIP call),
// kernel choice by M, launches, and the host-only block-32 scale packer.

#include <math.h>
#include <string.h>

#include <atomic>
#include <mutex>

#include "bfp8.h"
#include "bfp8_launch.hpp"
#include "stream_common.hpp"

using namespace bfp8;

namespace {

constexpr int64_t kAlign = 16;
constexpr int64_t kMaxDim = (int64_t)1 << 31;   // every size must fit the kernels' 32-bit grid math

bool aligned(const void* p) { return ((uintptr_t)p % kAlign) == 0; }
bool dim_ok(int64_t v, int64_t lo) { return v >= lo && v < kMaxDim; }
bool is16(int dtype) { return dtype == BFP8_BF16 || dtype == BFP8_F16; }
bool is_out(int dtype) { return dtype == BFP8_BF16 || dtype == BFP8_F16 || dtype == BFP8_F32; }
hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }
bfp8_status launched(hipError_t e) { return e == hipSuccess ? BFP8_OK : BFP8_E_LAUNCH; }

// Checks shared by the three GEMMs; `k_mult` / `n_mult` are the op's shape rules.
bfp8_status check_gemm(const void* a, const void* b, const void* c, const void* y, int y_dtype,
                       int64_t M, int64_t N, int64_t K, int64_t n_mult, size_t need,
                       const void* workspace, size_t workspace_bytes) {
    if (!a || !b || !c || !y) return BFP8_E_NULL;
    if (!dim_ok(M, 1) || !dim_ok(N, n_mult) || !dim_ok(K, 128)) return BFP8_E_SHAPE;
    if (N % n_mult != 0 || K % 128 != 0 || K > kTileMaxK) return BFP8_E_SHAPE;
    if (M * K >= ((int64_t)1 << 40) || N * K >= ((int64_t)1 << 40)) return BFP8_E_SHAPE;
    if (!is_out(y_dtype)) return BFP8_E_DTYPE;
    if (!aligned(a) || !aligned(b) || !aligned(c) || !aligned(y)) return BFP8_E_ALIGN;
    if (need > 0) {
        if (!workspace || workspace_bytes < need) return BFP8_E_WORKSPACE;
        if (!aligned(workspace)) return BFP8_E_ALIGN;
    }
    return BFP8_OK;
}

}  // namespace

extern "C" {

bfp8_status bfp8_quantize_act_1x128(const void* x, int x_dtype, int64_t M, int64_t K,
                                    uint8_t* xq, float* xs, void* stream) {
    if (!x || !xq || !xs) return BFP8_E_NULL;
    if (!dim_ok(M, 1) || !dim_ok(K, 8) || K % 8 != 0 || M * K >= ((int64_t)1 << 40)) return BFP8_E_SHAPE;
    if (M * ((K + 2047) / 2048) >= kMaxDim) return BFP8_E_SHAPE;   // one workgroup per row and 2048 columns
    if (!is16(x_dtype)) return BFP8_E_DTYPE;
    if (!aligned(x) || !aligned(xq) || !aligned(xs)) return BFP8_E_ALIGN;
    return launched(launch_quant_act_1x128(x, x_dtype == BFP8_BF16, M, K, xq, xs, as_stream(stream)));
}

bfp8_status bfp8_quantize_weight_128x128(const void* w, int w_dtype, int64_t N, int64_t K,
                                         uint8_t* wq, float* ws, void* stream) {
    if (!w || !wq || !ws) return BFP8_E_NULL;
    if (!dim_ok(N, 1) || !dim_ok(K, 8) || K % 8 != 0 || N * K >= ((int64_t)1 << 40)) return BFP8_E_SHAPE;
    if ((N + 127) / 128 > 65535) return BFP8_E_SHAPE;      // grid.y limit
    if (!is16(w_dtype)) return BFP8_E_DTYPE;
    if (!aligned(w) || !aligned(wq) || !aligned(ws)) return BFP8_E_ALIGN;
    return launched(launch_quant_weight_128x128(w, w_dtype == BFP8_BF16, N, K, wq, ws, as_stream(stream)));
}

bfp8_status bfp8_dequantize_weight(const uint8_t* wq, const float* scales, int64_t block, void* w, int w_dtype,
                                   int64_t N, int64_t K, void* stream) {
    if (!wq || !scales || !w) return BFP8_E_NULL;
    if (block != 32 && block != 128) return BFP8_E_SHAPE;
    if (!dim_ok(N, 1) || !dim_ok(K, 8) || K % 8 != 0 || N * K >= ((int64_t)1 << 40)) return BFP8_E_SHAPE;
    if (N * ((K + 2047) / 2048) >= kMaxDim) return BFP8_E_SHAPE;   // one workgroup per row and 2048 columns
    if (!is_out(w_dtype)) return BFP8_E_DTYPE;
    if (!aligned(wq) || !aligned(scales) || !aligned(w)) return BFP8_E_ALIGN;
    return launched(launch_dequant_weight(wq, scales, (int)block, w, w_dtype, N, K, as_stream(stream)));
}

}  // extern "C"

namespace {

size_t round256(size_t v) { return (v + 255) / 256 * 256; }

// The fused quantise + W8A8 call quantises inside the kernel when the codes
// call would run the one-token kernel or stream (so both give the same
// bits), M permitting.
bool quantises_in_registers(int64_t M, int64_t N, int64_t K) {
    return one_token(M, K) || (M <= kFusedQuantMaxM && w8a8_streams(M, N, K));
}

// The kernel each GEMM op runs for a shape: the one routing rule behind the
// launches below and bfp8_get_plan.  For the fused quantise + W8A8 op
// outside the in-kernel range this is the W8A8 kernel that follows the
// staged quantiser.
int route(int op, int64_t M, int64_t N, int64_t K) {
    switch (op) {
        case BFP8_OP_QUANT_GEMM_W8A8_BLK128:
            if (one_token(M, K)) return BFP8_KERNEL_W8A8_GEMV_QUANT;
            if (quantises_in_registers(M, N, K)) return BFP8_KERNEL_W8A8_STREAM_QUANT;
            return route(BFP8_OP_GEMM_W8A8_BLK128, M, N, K);
        case BFP8_OP_GEMM_W8A8_BLK128:
            if (one_token(M, K)) return BFP8_KERNEL_W8A8_GEMV;
            if (w8a8_streams(M, N, K)) return BFP8_KERNEL_W8A8_STREAM;
            if (w8a8_wide(M, N, K)) return BFP8_KERNEL_W8A8_WIDE;
            return BFP8_KERNEL_W8A8_TILE;
        case BFP8_OP_GEMM_W8A16_BLK128:
            if (one_token_w8a16(M, K)) return BFP8_KERNEL_W8A16_GEMV;
            if (w8a16_wide(M, N, K)) return BFP8_KERNEL_W8A16_WIDE;
            if (M > kStreamMaxM) return BFP8_KERNEL_W8A16_TILE;
            return BFP8_KERNEL_W8A16_STREAM;
        case BFP8_OP_GEMM_W8A16_BLK32_UE8M0:
            if (one_token(M, K)) return BFP8_KERNEL_BLK32_GEMV;
            if (blk32_tile(M, N, K)) return BFP8_KERNEL_BLK32_TILE;
            if (blk32_wide(M, N, K)) return BFP8_KERNEL_BLK32_WIDE;
            return M <= kStreamMaxM ? BFP8_KERNEL_BLK32_STREAM_LDS : BFP8_KERNEL_BLK32_STREAM;
        case BFP8_OP_QUANT_ACT_1X128:
            return BFP8_KERNEL_QUANT_ACT;
        case BFP8_OP_QUANT_WEIGHT_128X128:
            return BFP8_KERNEL_QUANT_WEIGHT;
        default:
            return BFP8_KERNEL_NONE;
    }
}


// Workspace of the kernel route() picks (the launches use the same route,
// so the size always matches what the launched kernel uses): the streaming
// or tiled plan's split-K counters and partial tiles, none otherwise.
size_t kernel_workspace(int kernel, int64_t M, int64_t N, int64_t K) {
    switch (kernel) {
        case BFP8_KERNEL_W8A8_STREAM:
        case BFP8_KERNEL_W8A8_STREAM_QUANT:
        case BFP8_KERNEL_W8A16_STREAM:
        case BFP8_KERNEL_BLK32_STREAM_LDS:
        case BFP8_KERNEL_BLK32_STREAM:
            return stream_workspace_bytes(plan_stream(M, N, K));
        case BFP8_KERNEL_W8A8_TILE:
            return K <= kTileMaxK ? tile_workspace_bytes(M, N, K) : 0;
        case BFP8_KERNEL_W8A8_WIDE:
            return w8a8_wide_workspace_bytes(w8a8_wide_shape(M, N, K));
        case BFP8_KERNEL_W8A16_TILE:
        case BFP8_KERNEL_BLK32_TILE:
            return K <= kTileMaxK ? tile16_workspace_bytes(M, N, K) : 0;
        default:
            return 0;
    }
}

size_t w8a8_workspace(int64_t M, int64_t N, int64_t K) {
    return kernel_workspace(route(BFP8_OP_GEMM_W8A8_BLK128, M, N, K), M, N, K);
}

// The W8A8 codes kernels by M (workspace already checked).
hipError_t launch_w8a8(const uint8_t* xq, const float* xs, const uint8_t* wq, const float* ws, void* y,
                       int y_dtype, int64_t M, int64_t N, int64_t K, void* workspace, hipStream_t stream) {
    switch (route(BFP8_OP_GEMM_W8A8_BLK128, M, N, K)) {
        case BFP8_KERNEL_W8A8_GEMV: return launch_w8a8_gemv(xq, xs, wq, ws, y, y_dtype, N, K, stream);
        case BFP8_KERNEL_W8A8_STREAM:
            return launch_w8a8_stream(xq, xs, wq, ws, y, y_dtype, M, N, K, workspace, stream);
        case BFP8_KERNEL_W8A8_WIDE: return launch_w8a8_wide(xq, xs, wq, ws, y, y_dtype, M, N, K, workspace, stream);
        default: return launch_w8a8_tile(xq, xs, wq, ws, y, y_dtype, M, N, K, workspace, stream);
    }
}

// Workspace of the fused quantise + W8A8 call when it does not, where
// the codes are staged: [W8A8 workspace | xq codes M*K | xs scales M*K/128],
// each part 256-byte aligned, the zero-initialised counters first.
struct QuantGemmParts {
    size_t gemm, xq, xs, total;
};
QuantGemmParts quant_gemm_parts(int64_t M, int64_t N, int64_t K) {
    QuantGemmParts p;
    p.gemm = round256(w8a8_workspace(M, N, K));
    p.xq = round256((size_t)(M * K));
    p.xs = round256((size_t)(M * (K / 128)) * sizeof(float));
    p.total = p.gemm + p.xq + p.xs;
    return p;
}

}  // namespace

extern "C" {

size_t bfp8_workspace_bytes(int op, int64_t M, int64_t N, int64_t K) {
    if (M < 1 || N < 16 || K < 128) return 0;
    switch (op) {
        case BFP8_OP_QUANT_GEMM_W8A8_BLK128: {
            const int kernel = route(op, M, N, K);
            if (kernel == BFP8_KERNEL_W8A8_GEMV_QUANT || kernel == BFP8_KERNEL_W8A8_STREAM_QUANT)
                return kernel_workspace(kernel, M, N, K);
            return K <= kTileMaxK ? quant_gemm_parts(M, N, K).total : 0;   // codes staged by the quantiser
        }
        case BFP8_OP_GEMM_W8A8_BLK128:
        case BFP8_OP_GEMM_W8A16_BLK128:
        case BFP8_OP_GEMM_W8A16_BLK32_UE8M0:
            return kernel_workspace(route(op, M, N, K), M, N, K);
        default:
            return 0;
    }
}

bfp8_status bfp8_gemm_w8a8_blk128(const uint8_t* xq, const float* xs, const uint8_t* wq, const float* ws,
                                  void* y, int y_dtype, int64_t M, int64_t N, int64_t K,
                                  void* workspace, size_t workspace_bytes, void* stream) {
    if (!xq || !xs || !wq || !ws || !y) return BFP8_E_NULL;
    const size_t need = (dim_ok(M, 1) && dim_ok(N, 16) && dim_ok(K, 128))
                            ? bfp8_workspace_bytes(BFP8_OP_GEMM_W8A8_BLK128, M, N, K) : 0;
    bfp8_status st = check_gemm(xq, wq, ws, y, y_dtype, M, N, K, 16, need, workspace, workspace_bytes);
    if (st != BFP8_OK) return st;
    if (!aligned(xs)) return BFP8_E_ALIGN;
    return launched(launch_w8a8(xq, xs, wq, ws, y, y_dtype, M, N, K, workspace, as_stream(stream)));
}

}  // extern "C"

// ------------------------------------------------ allocation-free variant ----
// bfp8_gemm_w8a8_blk128_noalloc takes its workspace from this array: one
// copy per GPU, held by the loaded library until the process ends.  Host code
// never uses the array's name as a device address (in host code it names a
// host-side stand-in); the device address comes from hipGetSymbolAddress,
// once per device, and only that pointer is passed to kernels.
namespace {

static __device__ __attribute__((aligned(256))) uint8_t scratch[BFP8_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// The scratch address on the current device (set up on its first use).
hipError_t scratch_on_current_device(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    void* p = g_scratch[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch[dev].load(std::memory_order_relaxed);
        if (!p) {
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess) return e;
            if (!p) return hipErrorInvalidSymbol;
            g_scratch[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return hipSuccess;
}

// Clears n dwords with vector stores (a kernel, not a memset, so the call
// can be captured into a HIP graph).
__global__ __launch_bounds__(256) void clear_words_kernel(uint32_t* __restrict__ p, uint32_t n) {
    for (uint32_t i = blockIdx.x * 256u + threadIdx.x; i < n; i += gridDim.x * 256u) p[i] = 0u;
}

// Leading workspace bytes of the W8A8 codes call that must be zero when it
// starts: the split-K tile counters of its plan (0 when it does not split K).
size_t w8a8_counter_bytes(int64_t M, int64_t N, int64_t K) {
    switch (route(BFP8_OP_GEMM_W8A8_BLK128, M, N, K)) {
        case BFP8_KERNEL_W8A8_STREAM: {
            const StreamPlan p = plan_stream(M, N, K);
            return p.splits > 1 ? stream_counter_bytes(p) : 0;
        }
        case BFP8_KERNEL_W8A8_TILE:
            return tile_counter_bytes(M, N, K);
        case BFP8_KERNEL_W8A8_WIDE:
            return w8a8_wide_counter_bytes(w8a8_wide_shape(M, N, K));
        default:
            return 0;
    }
}

}  // namespace

extern "C" {

bfp8_status bfp8_gemm_w8a8_blk128_noalloc(const uint8_t* xq, const float* xs, const uint8_t* wq, const float* ws,
                                          void* y, int y_dtype, int64_t M, int64_t N, int64_t K, void* stream) {
    if (!xq || !xs || !wq || !ws || !y) return BFP8_E_NULL;
    const size_t need = (dim_ok(M, 1) && dim_ok(N, 16) && dim_ok(K, 128))
                            ? bfp8_workspace_bytes(BFP8_OP_GEMM_W8A8_BLK128, M, N, K) : 0;
    bfp8_status st = check_gemm(xq, wq, ws, y, y_dtype, M, N, K, 16, 0, nullptr, 0);
    if (st != BFP8_OK) return st;
    if (!aligned(xs)) return BFP8_E_ALIGN;
    if (need > BFP8_NOALLOC_SCRATCH_BYTES) return BFP8_E_WORKSPACE;
    void* work = nullptr;
    if (need > 0) {
        if (scratch_on_current_device(&work) != hipSuccess) return BFP8_E_LAUNCH;
        const size_t counters = w8a8_counter_bytes(M, N, K);
        if (counters > 0) {
            const uint32_t words = (uint32_t)(counters / 4);
            hipLaunchKernelGGL(clear_words_kernel, dim3((words + 255) / 256), dim3(256), 0, as_stream(stream),
                               static_cast<uint32_t*>(work), words);
            if (hipGetLastError() != hipSuccess) return BFP8_E_LAUNCH;
        }
    }
    return launched(launch_w8a8(xq, xs, wq, ws, y, y_dtype, M, N, K, work, as_stream(stream)));
}

bfp8_status bfp8_quant_gemm_w8a8_blk128(const void* x, int x_dtype, const uint8_t* wq, const float* ws,
                                        void* y, int y_dtype, int64_t M, int64_t N, int64_t K,
                                        void* workspace, size_t workspace_bytes, void* stream) {
    if (!x || !wq || !ws || !y) return BFP8_E_NULL;
    const size_t need = (dim_ok(M, 1) && dim_ok(N, 16) && dim_ok(K, 128))
                            ? bfp8_workspace_bytes(BFP8_OP_QUANT_GEMM_W8A8_BLK128, M, N, K) : 0;
    bfp8_status st = check_gemm(x, wq, ws, y, y_dtype, M, N, K, 16, need, workspace, workspace_bytes);
    if (st != BFP8_OK) return st;
    if (!is16(x_dtype)) return BFP8_E_DTYPE;
    const int kernel = route(BFP8_OP_QUANT_GEMM_W8A8_BLK128, M, N, K);
    if (kernel == BFP8_KERNEL_W8A8_GEMV_QUANT)
        return launched(launch_w8a8_gemv_quant(x, x_dtype == BFP8_BF16, wq, ws, y, y_dtype, N, K, as_stream(stream)));
    if (kernel == BFP8_KERNEL_W8A8_STREAM_QUANT)
        return launched(launch_w8a8_stream_quant(x, x_dtype == BFP8_BF16, wq, ws, y, y_dtype, M, N, K, workspace,
                                                 as_stream(stream)));
    if (K > kTileMaxK) return BFP8_E_SHAPE;
    if (M * ((K + 2047) / 2048) >= kMaxDim) return BFP8_E_SHAPE;    // quantiser grid
    const QuantGemmParts parts = quant_gemm_parts(M, N, K);
    char* base = static_cast<char*>(workspace);
    uint8_t* xq = reinterpret_cast<uint8_t*>(base + parts.gemm);
    float* xs = reinterpret_cast<float*>(base + parts.gemm + parts.xq);
    void* gemm_ws = parts.gemm ? workspace : nullptr;
    hipError_t e = launch_quant_act_1x128(x, x_dtype == BFP8_BF16, M, K, xq, xs, as_stream(stream));
    if (e != hipSuccess) return BFP8_E_LAUNCH;
    return launched(launch_w8a8(xq, xs, wq, ws, y, y_dtype, M, N, K, gemm_ws, as_stream(stream)));
}

bfp8_status bfp8_gemm_w8a16_blk128(const void* x, int x_dtype, const uint8_t* wq, const float* ws,
                                   void* y, int y_dtype, int64_t M, int64_t N, int64_t K,
                                   void* workspace, size_t workspace_bytes, void* stream) {
    if (!x || !wq || !ws || !y) return BFP8_E_NULL;
    const size_t need = (dim_ok(M, 1) && dim_ok(N, 16) && dim_ok(K, 128))
                            ? bfp8_workspace_bytes(BFP8_OP_GEMM_W8A16_BLK128, M, N, K) : 0;
    bfp8_status st = check_gemm(x, wq, ws, y, y_dtype, M, N, K, 16, need, workspace, workspace_bytes);
    if (st != BFP8_OK) return st;
    if (!is16(x_dtype)) return BFP8_E_DTYPE;
    const bool bf = x_dtype == BFP8_BF16;
    switch (route(BFP8_OP_GEMM_W8A16_BLK128, M, N, K)) {
        case BFP8_KERNEL_W8A16_GEMV:    // one token: dot products on the vector ALUs
            return launched(launch_w8a16_gemv(x, bf, wq, ws, y, y_dtype, N, K, as_stream(stream)));
        case BFP8_KERNEL_W8A16_WIDE:    // every token per workgroup, weights widened in registers
            return launched(launch_w8a16_wide(x, bf, wq, ws, y, y_dtype, M, N, K, as_stream(stream)));
        case BFP8_KERNEL_W8A16_TILE:    // tiled MFMA kernel, weights widened in registers
            return launched(launch_w8a16_tile(x, bf, wq, ws, y, y_dtype, M, N, K, workspace, as_stream(stream)));
        default:
            return launched(launch_w8a16_blk128_stream(x, bf, wq, ws, y, y_dtype, M, N, K, workspace,
                                                       as_stream(stream)));
    }
}

bfp8_status bfp8_gemm_w8a16_blk32_ue8m0(const void* x, int x_dtype, const uint8_t* wq, const uint8_t* e8m0,
                                        void* y, int y_dtype, int64_t M, int64_t N, int64_t K,
                                        void* workspace, size_t workspace_bytes, void* stream) {
    if (!x || !wq || !e8m0 || !y) return BFP8_E_NULL;
    const size_t need = (dim_ok(M, 1) && dim_ok(N, 32) && dim_ok(K, 128))
                            ? bfp8_workspace_bytes(BFP8_OP_GEMM_W8A16_BLK32_UE8M0, M, N, K) : 0;
    bfp8_status st = check_gemm(x, wq, e8m0, y, y_dtype, M, N, K, 32, need, workspace, workspace_bytes);
    if (st != BFP8_OK) return st;
    if (x_dtype != BFP8_F16) return BFP8_E_DTYPE;
    if ((M + 15) / 16 > 65535) return BFP8_E_SHAPE;
    switch (route(BFP8_OP_GEMM_W8A16_BLK32_UE8M0, M, N, K)) {
        case BFP8_KERNEL_BLK32_GEMV:   // one token: dot products on the vector ALUs
            return launched(launch_w8a16_blk32_gemv(x, wq, e8m0, y, y_dtype, N, K, as_stream(stream)));
        case BFP8_KERNEL_BLK32_WIDE:   // M > 8: all tokens of a group per weight tile, rows through LDS
            return launched(launch_w8a16_blk32_wide(x, wq, e8m0, y, y_dtype, M, N, K, as_stream(stream)));
        case BFP8_KERNEL_BLK32_TILE:   // tiled MFMA kernel, scales applied in the widening
            return launched(launch_w8a16_blk32_tile(x, wq, e8m0, y, y_dtype, M, N, K, workspace, as_stream(stream)));
        default:
            return launched(launch_w8a16_blk32_stream(x, wq, e8m0, y, y_dtype, M, N, K, workspace,
                                                      as_stream(stream)));
    }
}

bfp8_status bfp8_prepare_blk32_ue8m0(const uint8_t* wq_host, const float* scale_host, int64_t N, int64_t K,
                                     uint8_t* e8m0_host, int64_t* bad_index) {
    if (bad_index) *bad_index = -1;
    if (!wq_host || !scale_host || !e8m0_host || !bad_index) return BFP8_E_NULL;
    // N in 32-row tiles; K in whole 128-K blocks, the unit the block-32 GEMM
    // streams (so a layer this packer accepts is one the GEMM accepts).
    if (N < 32 || K < 128 || N % 32 != 0 || K % 128 != 0 || N >= kMaxDim || K >= kMaxDim) return BFP8_E_SHAPE;
    const int64_t count = N * K;
    for (int64_t i = 0; i < count; ++i) {
        if ((wq_host[i] & 0x7F) == 0x7F) {
            *bad_index = i;
            return BFP8_E_NAN_CODE;
        }
    }
    const int64_t scales = (N / 32) * (K / 32);
    for (int64_t i = 0; i < scales; ++i) {
        const float s = scale_host[i];
        if (!isfinite(s) || !(s > 0.0f)) {
            *bad_index = i;
            return BFP8_E_SCALE_NOT_POW2;
        }
        int e2 = 0;
        const float frac = frexpf(s, &e2);         // s = frac * 2^e2, frac in [0.5, 1), exact
        if (frac != 0.5f) {
            *bad_index = i;
            return BFP8_E_SCALE_NOT_POW2;
        }
        const int e = e2 - 1;
        if (e < -14 || e > 7) {
            *bad_index = i;
            return BFP8_E_SCALE_WINDOW;
        }
    }
    for (int64_t i = 0; i < scales; ++i) {
        int e2 = 0;
        frexpf(scale_host[i], &e2);
        e8m0_host[i] = (uint8_t)(e2 - 1 + 127);
    }
    return BFP8_OK;
}

bfp8_status bfp8_get_limits(int op, int64_t* k_multiple, int64_t* n_multiple, int64_t* align_bytes,
                            int64_t* m_stream_max) {
    int64_t k = 0, n = 0, ms = 0;
    switch (op) {
        case BFP8_OP_QUANT_ACT_1X128: k = 8; n = 1; ms = 0; break;
        case BFP8_OP_QUANT_WEIGHT_128X128: k = 8; n = 1; ms = 0; break;
        case BFP8_OP_GEMM_W8A8_BLK128: k = 128; n = 16; ms = kStreamMaxM; break;
        case BFP8_OP_QUANT_GEMM_W8A8_BLK128: k = 128; n = 16; ms = kStreamMaxM; break;
        case BFP8_OP_GEMM_W8A16_BLK128: k = 128; n = 16; ms = kStreamMaxM; break;
        case BFP8_OP_GEMM_W8A16_BLK32_UE8M0: k = 128; n = 32; ms = INT32_MAX; break;
        default: return BFP8_E_OP;
    }
    if (k_multiple) *k_multiple = k;
    if (n_multiple) *n_multiple = n;
    if (align_bytes) *align_bytes = kAlign;
    if (m_stream_max) *m_stream_max = ms;
    return BFP8_OK;
}

bfp8_status bfp8_get_plan(int op, int64_t M, int64_t N, int64_t K, bfp8_plan* plan) {
    if (!plan) return BFP8_E_NULL;
    if (op < BFP8_OP_QUANT_ACT_1X128 || op > BFP8_OP_QUANT_GEMM_W8A8_BLK128) return BFP8_E_OP;
    bfp8_plan p;
    memset(&p, 0, sizeof(p));
    p.kernel = route(op, M, N, K);
    p.splits = 1;
    if (op == BFP8_OP_QUANT_ACT_1X128 || op == BFP8_OP_QUANT_WEIGHT_128X128) {
        // The quantisers take their own shape rules (N stands for the weight rows).
        const int64_t rows = op == BFP8_OP_QUANT_ACT_1X128 ? M : N;
        if (!dim_ok(rows, 1) || !dim_ok(K, 8) || K % 8 != 0 || rows * K >= ((int64_t)1 << 40)) return BFP8_E_SHAPE;
        p.tile_n = op == BFP8_OP_QUANT_ACT_1X128 ? 0 : 128;
        p.waves = kQuantLaunchWaves;
        p.workgroups = op == BFP8_OP_QUANT_ACT_1X128 ? quant_act_workgroups(rows, K)
                                                     : ((rows + 127) / 128) * ((K + 127) / 128);
        *plan = p;
        return BFP8_OK;
    }
    const int64_t n_mult = op == BFP8_OP_GEMM_W8A16_BLK32_UE8M0 ? 32 : 16;
    if (!dim_ok(M, 1) || !dim_ok(N, n_mult) || !dim_ok(K, 128) || N % n_mult != 0 || K % 128 != 0 ||
        K > kTileMaxK || M * K >= ((int64_t)1 << 40) || N * K >= ((int64_t)1 << 40))
        return BFP8_E_SHAPE;
    if (op == BFP8_OP_GEMM_W8A16_BLK32_UE8M0 && (M + 15) / 16 > 65535) return BFP8_E_SHAPE;
    p.workspace_bytes = bfp8_workspace_bytes(op, M, N, K);
    if (op == BFP8_OP_QUANT_GEMM_W8A8_BLK128 && p.kernel != BFP8_KERNEL_W8A8_GEMV_QUANT &&
        p.kernel != BFP8_KERNEL_W8A8_STREAM_QUANT)
        p.quant_kernel = BFP8_KERNEL_QUANT_ACT;
    switch (p.kernel) {
        case BFP8_KERNEL_W8A8_GEMV:
        case BFP8_KERNEL_W8A16_GEMV:
        case BFP8_KERNEL_BLK32_GEMV: {
            p.tile_n = kGemvLaunchWaves;   // one weight row per wave
            p.tile_m = 1;
            p.waves = kGemvLaunchWaves;
            p.workgroups = (N + p.tile_n - 1) / p.tile_n;
            break;
        }
        case BFP8_KERNEL_W8A8_GEMV_QUANT:   // one weight row per wave
            p.tile_n = kGemvLaunchWaves;
            p.tile_m = 1;
            p.waves = kGemvLaunchWaves;
            p.workgroups = N / kGemvLaunchWaves;
            break;
        case BFP8_KERNEL_W8A8_STREAM:
        case BFP8_KERNEL_W8A8_STREAM_QUANT:
        case BFP8_KERNEL_W8A16_STREAM:
        case BFP8_KERNEL_BLK32_STREAM_LDS:
        case BFP8_KERNEL_BLK32_STREAM: {
            const StreamPlan sp = plan_stream(M, N, K);
            p.tile_n = (int)kStreamRows;
            p.tile_m = 16;
            p.waves = kStreamLaunchWaves;
            p.splits = (int)sp.splits;
            const bool z_tiles = p.kernel == BFP8_KERNEL_W8A8_STREAM || p.kernel == BFP8_KERNEL_BLK32_STREAM;
            p.workgroups = sp.n_tiles * sp.splits * (z_tiles ? sp.m_tiles : 1);
            break;
        }
        case BFP8_KERNEL_W8A8_WIDE:
        case BFP8_KERNEL_W8A16_WIDE:
        case BFP8_KERNEL_BLK32_WIDE: {
            const WideShape w = p.kernel == BFP8_KERNEL_W8A8_WIDE   ? w8a8_wide_shape(M, N, K)
                                : p.kernel == BFP8_KERNEL_BLK32_WIDE ? blk32_wide_shape(M, N)
                                                                     : w16_wide_shape(M, N);
            p.tile_n = 16 * w.kr;
            p.tile_m = 16 * w.kt;
            p.waves = p.kernel == BFP8_KERNEL_W8A8_WIDE ? w8a8_wide_waves(w.kr, w.kt) : w16_wide_waves(w.kr, w.kt);
            p.splits = w.splits;
            p.workgroups = (int64_t)w.groups_n * w.groups_m * w.splits;
            break;
        }
        case BFP8_KERNEL_W8A8_TILE:
        case BFP8_KERNEL_W8A16_TILE:
        case BFP8_KERNEL_BLK32_TILE: {
            const TileInfo t = p.kernel == BFP8_KERNEL_W8A8_TILE ? tile_info(M, N, K) : tile16_info(M, N, K);
            p.tile_n = t.tile_n;
            p.tile_m = t.tile_m;
            p.waves = t.waves;
            p.splits = (int)t.splits;
            p.workgroups = t.tiles * t.splits;
            break;
        }
        default:
            return BFP8_E_OP;
    }
    *plan = p;
    return BFP8_OK;
}

const char* bfp8_kernel_name(int kernel) {
    switch (kernel) {
        case BFP8_KERNEL_NONE: return "none";
        case BFP8_KERNEL_QUANT_ACT: return "quant_act_1x128";
        case BFP8_KERNEL_QUANT_WEIGHT: return "quant_weight_128x128";
        case BFP8_KERNEL_W8A8_GEMV: return "w8a8_gemv";
        case BFP8_KERNEL_W8A8_GEMV_QUANT: return "w8a8_gemv_quant";
        case BFP8_KERNEL_W8A8_STREAM: return "w8a8_stream";
        case BFP8_KERNEL_W8A8_STREAM_QUANT: return "w8a8_stream_quant";
        case BFP8_KERNEL_W8A8_WIDE: return "w8a8_wide";
        case BFP8_KERNEL_W8A8_TILE: return "w8a8_tile";
        case BFP8_KERNEL_W8A16_GEMV: return "w8a16_gemv";
        case BFP8_KERNEL_W8A16_STREAM: return "w8a16_stream";
        case BFP8_KERNEL_W8A16_WIDE: return "w8a16_wide";
        case BFP8_KERNEL_W8A16_TILE: return "w8a16_tile";
        case BFP8_KERNEL_BLK32_STREAM_LDS: return "blk32_stream_lds";
        case BFP8_KERNEL_BLK32_STREAM: return "blk32_stream";
        case BFP8_KERNEL_BLK32_GEMV: return "blk32_gemv";
        case BFP8_KERNEL_BLK32_WIDE: return "blk32_wide";
        case BFP8_KERNEL_BLK32_TILE: return "blk32_tile";
        default: return "unknown kernel";
    }
}

const char* bfp8_status_string(bfp8_status s) {
    switch (s) {
        case BFP8_OK: return "ok";
        case BFP8_E_NULL: return "a required pointer is NULL";
        case BFP8_E_SHAPE: return "a size is out of range or not a required multiple";
        case BFP8_E_DTYPE: return "unsupported dtype code";
        case BFP8_E_ALIGN: return "a device pointer is not 16-byte aligned";
        case BFP8_E_WORKSPACE: return "workspace missing or too small";
        case BFP8_E_NAN_CODE: return "E4M3 NaN code (0x7F/0xFF) in the weights";
        case BFP8_E_SCALE_NOT_POW2: return "block scale is not a positive finite power of two";
        case BFP8_E_SCALE_WINDOW: return "power-of-two scale outside [2^-14, 2^7]";
        case BFP8_E_LAUNCH: return "HIP kernel launch failed";
        case BFP8_E_OP: return "unknown op code";
        default: return "unknown status";
    }
}

}  // extern "C"
