// Shared pieces of the weight-streaming (M <= 16 per token tile) kernels:
// the cross-wave reduction of a 16x16 output tile in LDS, the deterministic
// split-K finish, and the output store.
//
// A streaming workgroup owns one 16-row tile of W (rows n) and one 16-token
// tile of X (columns m).  Its waves take disjoint 128-K blocks; each wave
// ends with a 16x16 fp32 tile in the MFMA output layout (lane l, register i
// holds row 4*(l/16)+i, column l%16).  The waves' tiles are summed in LDS in
// wave order.  With split-K, each of `splits` workgroups writes its tile to
// the workspace, and the last one to arrive (device-scope counter) sums all
// of them in split order, stores Y and re-arms the counter.  No
// floating-point atomics: results are run-to-run identical.
//
// The hand-off uses agent-scope relaxed atomic accesses (write-through
// stores and loads that bypass the per-XCD L2, and a memory-side atomic
// counter) plus explicit completion waits, not __threadfence(): on this part
// a device-scope fence writes back and invalidates the XCD's whole L2, which
// made a split-K call cost tens of microseconds.  Ordering: every thread's
// partial store has completed (vmcnt 0) before the workgroup barrier that
// precedes the counter increment, so a workgroup that sees the final count
// reads complete partial tiles.
#pragma once

#include "bfp8_device.hpp"
#include "bfp8_launch.hpp"

namespace bfp8 {

constexpr int kStreamWaves = 16;
constexpr int kStreamThreads = kStreamWaves * kWave;

// Workspace layout of a split-K plan: one uint32 counter per output tile
// (padded to 256 bytes), then splits fp32 16x16 tiles per output tile.
inline size_t stream_counter_bytes(const StreamPlan& p) {
    return ((size_t)(p.n_tiles * p.m_tiles) * sizeof(uint32_t) + 255) / 256 * 256;
}
inline void stream_workspace_parts(const StreamPlan& p, void* ws, uint32_t*& counters, float*& partials) {
    counters = nullptr;
    partials = nullptr;
    if (p.splits == 1) return;
    counters = static_cast<uint32_t*>(ws);
    partials = reinterpret_cast<float*>(static_cast<char*>(ws) + stream_counter_bytes(p));
}

__device__ __forceinline__ void store_out(void* y, int y_dtype, int64_t idx, float v) {
    if (y_dtype == 2) {
        static_cast<float*>(y)[idx] = v;
    } else if (y_dtype == 0) {
        static_cast<uint16_t*>(y)[idx] = (uint16_t)float_to_bf16_bits(v);
    } else {
        static_cast<uint16_t*>(y)[idx] = (uint16_t)float_to_f16_bits(v);
    }
}

// red: LDS scratch of kStreamWaves * 256 floats.  Must be called by every
// thread of the workgroup (it contains barriers).
__device__ __forceinline__ void stream_finish(f32x4 acc, float* red, void* y, int y_dtype,
                                              int64_t M, int64_t N, int64_t nt, int64_t mt,
                                              int64_t splits, int64_t split, int64_t n_tiles,
                                              float* partials, uint32_t* counters) {
    const int t = threadIdx.x;
    const int wave = t / kWave, lane = t % kWave;
#pragma unroll
    for (int i = 0; i < 4; ++i) red[wave * 256 + lane * 4 + i] = acc[i];
    __syncthreads();

    // Thread t < 256 owns output (m_loc = t / 16, n_loc = t % 16).
    const int m_loc = t >> 4, n_loc = t & 15;
    const int src = ((n_loc >> 2) * 16 + m_loc) * 4 + (n_loc & 3);
    float v = 0.0f;
    if (t < 256) {
#pragma unroll
        for (int w = 0; w < kStreamWaves; ++w) v += red[w * 256 + src];
    }
    const int64_t m = mt * 16 + m_loc;
    const int64_t n = nt * 16 + n_loc;

    if (splits == 1) {
        if (t < 256 && m < M) store_out(y, y_dtype, m * N + n, v);
        return;
    }

    const int64_t tile = mt * n_tiles + nt;
    float* my_tiles = partials + tile * splits * 256;
    if (t < 256) __hip_atomic_store(&my_tiles[split * 256 + t], v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __builtin_amdgcn_s_waitcnt(0);            // this thread's partial store has completed
    __syncthreads();
    __shared__ uint32_t arrived;
    if (t == 0) arrived = __hip_atomic_fetch_add(&counters[tile], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    if (arrived != (uint32_t)(splits - 1)) return;   // not the last workgroup of this tile

    if (t < 256) {
        // Sum in split order; the loads of eight splits are issued together
        // before any is added (one memory round trip per eight splits).
        constexpr int kChunk = 8;
        float s = 0.0f;
        for (int64_t k0 = 0; k0 < splits; k0 += kChunk) {
            float p[kChunk];
#pragma unroll
            for (int u = 0; u < kChunk; ++u)
                if (k0 + u < splits)
                    p[u] = __hip_atomic_load(&my_tiles[(k0 + u) * 256 + t], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
            for (int u = 0; u < kChunk; ++u)
                if (k0 + u < splits) s += p[u];
        }
        if (m < M) store_out(y, y_dtype, m * N + n, s);
    }
    if (t == 0) __hip_atomic_store(&counters[tile], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);   // re-arm
}

}  // namespace bfp8
