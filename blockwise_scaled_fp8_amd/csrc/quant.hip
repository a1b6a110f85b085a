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

// Grid: one workgroup per (row, run of 16 groups); 16 threads per group,
// one thread per 8 input values.
__global__ __launch_bounds__(kQuantActThreads) void quant_act_1x128_kernel(
    const uint16_t* __restrict__ x, int bf16, int64_t M, int64_t K, int64_t G, int64_t blocks_per_row,
    uint8_t* __restrict__ xq, float* __restrict__ xs) {
    // 32-bit index arithmetic (the launcher keeps the grid below 2^32): the
    // 64-bit division took some fifty scalar instructions per wave.
    const uint32_t mb = (uint32_t)blockIdx.x / (uint32_t)blocks_per_row;   // uniform per workgroup
    const int64_t m = mb;
    const int64_t g = (int64_t)((uint32_t)blockIdx.x - mb * (uint32_t)blocks_per_row) * (kQuantActThreads / 16) +
                      (threadIdx.x >> 4);
    const int lane16 = threadIdx.x & 15;
    const int64_t col = g * 128 + lane16 * 8;
    const bool valid = g < G && col < K;            // K % 8 == 0: a chunk is all in or all out

    const u32x4 raw = valid ? load_16B(x + m * K + col) : u32x4{0u, 0u, 0u, 0u};
    float v[8];
    unpack8(raw, bf16 != 0, v);
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
    amax = group16_max(amax);                       // all 16 lanes of a group are in one wave

    const float s = amax / 448.0f;
    uint32_t lo, hi;
    quantize8(v, raw, s, lo, hi);
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

hipError_t launch_quant_act_1x128(const void* x, bool bf16, int64_t M, int64_t K,
                                  uint8_t* xq, float* xs, hipStream_t stream) {
    const int64_t G = (K + 127) / 128;
    const int64_t blocks_per_row = (G + kQuantActThreads / 16 - 1) / (kQuantActThreads / 16);
    if (M * blocks_per_row >= (int64_t(1) << 32)) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(quant_act_1x128_kernel, dim3((unsigned)(M * blocks_per_row)), dim3(kQuantActThreads), 0,
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
