// Block quantisers: 1x128 activation groups and 128x128 weight tiles.
//
// [ARC] "Route-2 handover" item 3: the generic block quantiser ran 1024
// threads per 1x128 group with 31/32 of them idle and 128 serialised atomic
// maxima; the fix it names is one small lane group per 128 values, a
// register reduction and vector loads.  Here 16 lanes own one group, each
// lane loads its 8 values with one 16-byte load, the group maximum is a
// 4-step butterfly over the 16 lanes, and each lane writes its 8 codes with
// one 8-byte store.  A wave covers 4 groups.
//
// The scale is an IEEE fp32 division (the compiler's default, correctly
// rounded, fp32 division) and each element's quotient x / s is the correctly
// rounded fp32 quotient (QuotientBy: one IEEE division per group, three
// instructions per element), so the codes and scales are bit-exact functions
// of the input.

#include "bfp8_device.hpp"
#include "bfp8_launch.hpp"

namespace bfp8 {

constexpr int kQuantActThreads = 256;
constexpr int kQuantActRows = 2;   // token rows per thread

// Grid: one workgroup per (pair of rows, run of 16 groups); 16 threads per
// group, one thread per 8 input values of each of its two rows.  Both rows'
// loads are issued before either is quantised, and the codes are written
// with non-temporal stores (nothing reads them again before the GEMM):
// 11.4 -> 9.9 us at M = K = 4096 (one row per thread with ordinary stores
// before; four or eight rows per thread, or non-temporal loads, were slower).
__global__ __launch_bounds__(kQuantActThreads) void quant_act_1x128_kernel(
    const uint16_t* __restrict__ x, int bf16, int64_t M, int64_t K, int64_t G, int64_t blocks_per_row,
    uint8_t* __restrict__ xq, float* __restrict__ xs) {
    // 32-bit index arithmetic (the launcher keeps the grid below 2^32): the
    // 64-bit division took some fifty scalar instructions per wave.
    const uint32_t mb = (uint32_t)blockIdx.x / (uint32_t)blocks_per_row;   // uniform per workgroup
    const int64_t m0 = (int64_t)mb * kQuantActRows;
    const int64_t g = (int64_t)((uint32_t)blockIdx.x - mb * (uint32_t)blocks_per_row) * (kQuantActThreads / 16) +
                      (threadIdx.x >> 4);
    const int lane16 = threadIdx.x & 15;
    const int64_t col = g * 128 + lane16 * 8;
    const bool valid = g < G && col < K;            // K % 8 == 0: a chunk is all in or all out

    u32x4 raw[kQuantActRows];
#pragma unroll
    for (int r = 0; r < kQuantActRows; ++r)
        raw[r] = valid && m0 + r < M ? load_16B(x + (m0 + r) * K + col) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int r = 0; r < kQuantActRows; ++r) {
        const int64_t m = m0 + r;
        float v[8];
        unpack8(raw[r], bf16 != 0, v);
        float amax = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
        amax = group16_max(amax);                   // all 16 lanes of a group are in one wave

        const float s = amax / 448.0f;
        uint32_t lo, hi;
        quantize8(v, raw[r], s, lo, hi);
        if (valid && m < M) {
            __builtin_nontemporal_store(u32x2{lo, hi}, reinterpret_cast<u32x2*>(xq + m * K + col));
            if (lane16 == 0) xs[m * G + g] = s;
        }
    }
}

// One workgroup per 128x128 tile; thread t owns 8-column chunk (t % 16) of
// rows (t / 16) + 16 i, i = 0..7.
constexpr int kQuantWThreads = 256;

__global__ __launch_bounds__(kQuantWThreads) void quant_weight_128x128_kernel(
    const uint16_t* __restrict__ w, int bf16, int64_t N, int64_t K, int64_t KB,
    uint8_t* __restrict__ wq, float* __restrict__ ws) {
    __shared__ float wave_amax[kQuantWThreads / kWave];
    const int64_t nb = blockIdx.y, kb = blockIdx.x;
    const int t = threadIdx.x;
    const int64_t col = kb * 128 + (t & 15) * 8;
    const bool col_ok = col < K;

    float v[8][8];
    u32x4 raw[8];
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int64_t row = nb * 128 + (t >> 4) + 16 * i;
        raw[i] = col_ok && row < N ? load_16B(w + row * K + col) : u32x4{0u, 0u, 0u, 0u};
        unpack8(raw[i], bf16 != 0, v[i]);
#pragma unroll
        for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(v[i][j]));
    }
    amax = wave_max(amax);
    if ((t & (kWave - 1)) == 0) wave_amax[t / kWave] = amax;
    __syncthreads();
    amax = fmaxf(fmaxf(wave_amax[0], wave_amax[1]), fmaxf(wave_amax[2], wave_amax[3]));

    const float s = amax / 448.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int64_t row = nb * 128 + (t >> 4) + 16 * i;
        uint32_t lo, hi;
        quantize8(v[i], raw[i], s, lo, hi);
        if (col_ok && row < N) *reinterpret_cast<uint2*>(wq + row * K + col) = make_uint2(lo, hi);
    }
    if (t == 0) ws[nb * KB + kb] = s;
}

// Load-time blockwise dequantisation: w = RN_out(fl32(E4M3(q) * s)) with one
// fp32 scale per B x B block (B = 32 or 128), the fallback for layers whose
// 32x32 scales the block-32 packer refuses ([SM70] "Exactness").  One thread
// per 8 consecutive weights of a row (one 8-byte code load, one 16-byte
// store for 16-bit outputs, two for fp32); the 8 share one block scale since
// B is a multiple of 8.  The E4M3 decode is gfx950's fp8 -> fp32 conversion
// (exact: every finite E4M3 value is an fp32 value; NaN codes give NaN).
constexpr int kDequantThreads = 256;

__global__ __launch_bounds__(kDequantThreads) void dequant_weight_kernel(
    const uint8_t* __restrict__ wq, const float* __restrict__ scales, int block, void* __restrict__ w,
    int w_dtype, int64_t N, int64_t K, int64_t blocks_per_row) {
    const uint32_t n32 = (uint32_t)blockIdx.x / (uint32_t)blocks_per_row;   // uniform per workgroup
    const int64_t n = n32;
    const int64_t k = ((int64_t)((uint32_t)blockIdx.x - n32 * (uint32_t)blocks_per_row) * kDequantThreads +
                       threadIdx.x) * 8;
    if (k >= K) return;
    const int64_t KBs = (K + block - 1) / block;
    const float s = scales[(n / block) * KBs + k / block];
    const uint2 q = *reinterpret_cast<const uint2*>(wq + n * K + k);
    // The conversion's byte select is an immediate.
    const float p[8] = {__builtin_amdgcn_cvt_f32_fp8((int)q.x, 0) * s, __builtin_amdgcn_cvt_f32_fp8((int)q.x, 1) * s,
                        __builtin_amdgcn_cvt_f32_fp8((int)q.x, 2) * s, __builtin_amdgcn_cvt_f32_fp8((int)q.x, 3) * s,
                        __builtin_amdgcn_cvt_f32_fp8((int)q.y, 0) * s, __builtin_amdgcn_cvt_f32_fp8((int)q.y, 1) * s,
                        __builtin_amdgcn_cvt_f32_fp8((int)q.y, 2) * s, __builtin_amdgcn_cvt_f32_fp8((int)q.y, 3) * s};
    const int64_t idx = n * K + k;
    if (w_dtype == 2) {
        float* out = static_cast<float*>(w) + idx;
        *reinterpret_cast<f32x4*>(out) = f32x4{p[0], p[1], p[2], p[3]};
        *reinterpret_cast<f32x4*>(out + 4) = f32x4{p[4], p[5], p[6], p[7]};
    } else {
        uint32_t h[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) h[i] = w_dtype == 0 ? float_to_bf16_bits(p[i]) : float_to_f16_bits(p[i]);
        *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(w) + idx) =
            u32x4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
    }
}

hipError_t launch_dequant_weight(const uint8_t* wq, const float* scales, int block, void* w, int w_dtype,
                                 int64_t N, int64_t K, hipStream_t stream) {
    const int64_t blocks_per_row = (K / 8 + kDequantThreads - 1) / kDequantThreads;
    if (N * blocks_per_row >= (int64_t(1) << 32)) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(dequant_weight_kernel, dim3((unsigned)(N * blocks_per_row)), dim3(kDequantThreads), 0, stream,
                       wq, scales, block, w, w_dtype, N, K, blocks_per_row);
    return hipGetLastError();
}

static_assert(kQuantActThreads == kQuantLaunchWaves * kWave && kQuantWThreads == kQuantLaunchWaves * kWave,
              "plan and launch agree");

int64_t quant_act_workgroups(int64_t M, int64_t K) {
    const int64_t G = (K + 127) / 128;
    return ((M + kQuantActRows - 1) / kQuantActRows) * ((G + kQuantActThreads / 16 - 1) / (kQuantActThreads / 16));
}

hipError_t launch_quant_act_1x128(const void* x, bool bf16, int64_t M, int64_t K,
                                  uint8_t* xq, float* xs, hipStream_t stream) {
    const int64_t G = (K + 127) / 128;
    const int64_t blocks_per_row = (G + kQuantActThreads / 16 - 1) / (kQuantActThreads / 16);
    const int64_t row_blocks = (M + kQuantActRows - 1) / kQuantActRows;
    if (row_blocks * blocks_per_row >= (int64_t(1) << 32)) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(quant_act_1x128_kernel, dim3((unsigned)(row_blocks * blocks_per_row)), dim3(kQuantActThreads), 0,
                       stream, static_cast<const uint16_t*>(x), (int)bf16, M, K, G, blocks_per_row, xq, xs);
    return hipGetLastError();
}

hipError_t launch_quant_weight_128x128(const void* w, bool bf16, int64_t N, int64_t K,
                                       uint8_t* wq, float* ws, hipStream_t stream) {
    const int64_t NB = (N + 127) / 128, KB = (K + 127) / 128;
    hipLaunchKernelGGL(quant_weight_128x128_kernel, dim3((unsigned)KB, (unsigned)NB), dim3(kQuantWThreads), 0,
                       stream, static_cast<const uint16_t*>(w), (int)bf16, N, K, KB, wq, ws);
    return hipGetLastError();
}

}  // namespace bfp8
