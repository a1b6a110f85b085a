// Streaming-read probe for the benchmark (not part of the GEMM library's
// C ABI): reads a buffer once with 16-byte loads and writes one dword per
// workgroup, so its time per launch is the floor that any kernel reading
// the same bytes in one launch faces on this GPU (launch, ramp-up and drain
// included).  Decode is bound by reading the weights once ([3090] §4.3: at
// batch 1 the DRAM stream is the whole cost), so the benchmark reports each
// decode kernel's time against this floor over the same rotated buffers.
//
// Each thread issues kLoads independent 16-byte loads before it combines
// any of them (all of a wave's loads are in flight together); consecutive
// lanes read consecutive 16 bytes, so each load instruction of a wave covers
// eight whole 128-byte lines.  The loads are non-temporal (nt), the policy
// that reads rotated copies fastest (4.42 vs 4.57 us for 16 MiB; sc0 or sc1
// alone: no change) and the one the decode kernels use for their weights.
// Bytes past `bytes` are not read (buffer descriptor range check).

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef int i32x4 __attribute__((ext_vector_type(4)));
constexpr int kThreads = 256;

template <int kLoads>
__global__ __launch_bounds__(kThreads) void read_probe_kernel(const uint8_t* __restrict__ src, uint32_t bytes,
                                                              uint32_t* __restrict__ sink) {
    const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(src), 0,
                                                                          (int)bytes, 0x00020000);
    const uint32_t base = (uint32_t)blockIdx.x * kThreads * 16 * kLoads + threadIdx.x * 16;
    i32x4 v[kLoads];
#pragma unroll
    for (int i = 0; i < kLoads; ++i)
        v[i] = __builtin_amdgcn_raw_buffer_load_b128(rsrc, (int)(base + i * kThreads * 16), 0, 2 /* nt */);
    int acc = 0;
#pragma unroll
    for (int i = 0; i < kLoads; ++i) acc ^= v[i][0] ^ v[i][1] ^ v[i][2] ^ v[i][3];
    // One dword per workgroup keeps the loads live; lane 0 of each wave
    // combines its wave's lanes first.
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) acc ^= __shfl_xor(acc, off, 64);
    __shared__ int part[kThreads / 64];
    if (threadIdx.x % 64 == 0) part[threadIdx.x / 64] = acc;
    __syncthreads();
    if (threadIdx.x == 0) sink[blockIdx.x] = (uint32_t)(part[0] ^ part[1] ^ part[2] ^ part[3]);
}

}  // namespace

extern "C" {

// Workgroups (and dwords of `sink`) a launch with `loads` loads per thread
// uses for `bytes` bytes; 0 for an unsupported `loads`.
int64_t bfp8_probe_workgroups(int64_t bytes, int loads) {
    if (loads != 4 && loads != 8 && loads != 16) return 0;
    const int64_t per = (int64_t)kThreads * 16 * loads;
    return (bytes + per - 1) / per;
}

// Reads `bytes` bytes at `src` (device, 16-byte aligned, bytes < 2^31) and
// writes bfp8_probe_workgroups(bytes, loads) dwords to `sink` (device).
// Returns 0, or -1 for bad arguments, or the HIP error of the launch.
int bfp8_read_probe(const void* src, int64_t bytes, int loads, uint32_t* sink, void* stream) {
    const int64_t wg = bfp8_probe_workgroups(bytes, loads);
    if (!src || !sink || wg == 0 || bytes <= 0 || bytes >= ((int64_t)1 << 31) || ((uintptr_t)src & 15)) return -1;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const uint8_t* p = static_cast<const uint8_t*>(src);
    const dim3 grid((unsigned)wg), block(kThreads);
    if (loads == 4) hipLaunchKernelGGL(read_probe_kernel<4>, grid, block, 0, s, p, (uint32_t)bytes, sink);
    else if (loads == 8) hipLaunchKernelGGL(read_probe_kernel<8>, grid, block, 0, s, p, (uint32_t)bytes, sink);
    else hipLaunchKernelGGL(read_probe_kernel<16>, grid, block, 0, s, p, (uint32_t)bytes, sink);
    return (int)hipGetLastError();
}

}  // extern "C"
