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
// The scale and the per-element quotient are IEEE fp32 divisions (the
// default, correctly rounded, fp32 division of the HIP compiler), so the
// codes and scales are bit-exact functions of the input.

#include "bfp8_device.hpp"
#include "bfp8_launch.hpp"

namespace bfp8 {

// Quantise 8 values against scale s; returns the 8 codes packed in K order.
__device__ __forceinline__ void quantize8(const float v[8], float s, uint32_t& lo, uint32_t& hi) {
    uint32_t c[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) c[i] = (s == 0.0f) ? 0u : e4m3_encode(v[i] / s);
    lo = c[0] | (c[1] << 8) | (c[2] << 16) | (c[3] << 24);
    hi = c[4] | (c[5] << 8) | (c[6] << 16) | (c[7] << 24);
}

__device__ __forceinline__ void unpack8(u32x4 raw, bool bf16, float v[8]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t w = raw[i];
        v[2 * i] = bf16 ? bf16_bits_to_float(w & 0xFFFFu) : f16_bits_to_float(w & 0xFFFFu);
        v[2 * i + 1] = bf16 ? bf16_bits_to_float(w >> 16) : f16_bits_to_float(w >> 16);
    }
}

constexpr int kQuantActThreads = 256;

// Grid: one thread per 8 input values of a group; 16 threads per group.
__global__ __launch_bounds__(kQuantActThreads) void quant_act_1x128_kernel(
    const uint16_t* __restrict__ x, int bf16, int64_t M, int64_t K, int64_t G,
    uint8_t* __restrict__ xq, float* __restrict__ xs) {
    const int64_t tid = (int64_t)blockIdx.x * kQuantActThreads + threadIdx.x;
    const int64_t group = tid >> 4;                 // flat (row, group) index
    const int lane16 = (int)(tid & 15);
    const bool group_valid = group < M * G;
    const int64_t m = group_valid ? group / G : 0;
    const int64_t g = group_valid ? group - m * G : 0;
    const int64_t col = g * 128 + lane16 * 8;
    const bool valid = group_valid && col < K;      // K % 8 == 0: a chunk is all in or all out

    float v[8];
    if (valid) {
        unpack8(load_16B(x + m * K + col), bf16 != 0, v);
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = 0.0f;
    }
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
    amax = group16_max(amax);                       // all 16 lanes of a group are in one wave

    const float s = amax / 448.0f;
    uint32_t lo, hi;
    quantize8(v, s, lo, hi);
    if (valid) {
        *reinterpret_cast<uint2*>(xq + m * K + col) = make_uint2(lo, hi);
        if (lane16 == 0) xs[m * G + g] = s;
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
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int64_t row = nb * 128 + (t >> 4) + 16 * i;
        if (col_ok && row < N) {
            unpack8(load_16B(w + row * K + col), bf16 != 0, v[i]);
        } else {
#pragma unroll
            for (int j = 0; j < 8; ++j) v[i][j] = 0.0f;
        }
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
        quantize8(v[i], s, lo, hi);
        if (col_ok && row < N) *reinterpret_cast<uint2*>(wq + row * K + col) = make_uint2(lo, hi);
    }
    if (t == 0) ws[nb * KB + kb] = s;
}

hipError_t launch_quant_act_1x128(const void* x, bool bf16, int64_t M, int64_t K,
                                  uint8_t* xq, float* xs, hipStream_t stream) {
    const int64_t G = (K + 127) / 128;
    const int64_t threads = M * G * 16;
    const int64_t blocks = (threads + kQuantActThreads - 1) / kQuantActThreads;
    hipLaunchKernelGGL(quant_act_1x128_kernel, dim3((unsigned)blocks), dim3(kQuantActThreads), 0, stream,
                       static_cast<const uint16_t*>(x), (int)bf16, M, K, G, xq, xs);
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
