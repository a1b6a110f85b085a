// W8A8 blockwise-scaled FP8 GEMM for gfx950.
//
//   for each 128-wide K block kb:
//     P[m, n]  = sum_{k in kb} E4M3(xq[m, k]) * E4M3(wq[n, k])      FP8 MFMA, fp32
//     Y[m, n] += P[m, n] * xs[m, kb] * ws[n / 128, kb]              once per block
//
// ([ADA] "The fix": MMA only inside the 128-wide block, one temporary per
// block and the scales applied once per block, which removed the spills of
// the per-slice version; [ARC] "What this adds": the K tile equals the scale
// block, so the scale is a single value per tile and block.)
//
// MI355X design.  The FP8 MFMA 16x16x128 consumes one whole 128-K scale
// block per instruction, so the block partial P of a 16x16 output tile is a
// single MFMA with a zero accumulator and the promotion is one fp32 FMA per
// output per block.  Tiles are oriented as Y^T: weight rows n are the MFMA
// row operand and tokens m the column operand, so each lane's four outputs
// share one token and one 128-row weight block and the combined scale
// xs[m, kb] * ws[n/128, kb] is a single value per lane per block; the four
// outputs are also four consecutive n of one row of Y, stored with one
// vector store.  The weight-scale row is taken per output column (here per
// 128-aligned tile), never once per workgroup of arbitrary width ([ADA]
// "The fix", the latent-bug paragraph).
//
// Two kernels, chosen by M ([ADA] "One tile doesn't fit all M"):
//   * stream (M <= 16): weight streaming.  One workgroup per 16 weight rows
//     (and per split of K), eight waves each holding several 128-K blocks of
//     weight loads in flight, tokens padded to 16 on the MFMA column axis.
//   * tile (M > 16): 128x128 output tiles, A and B staged through LDS with
//     16-byte global loads, double-buffered, four waves of 64x64 each,
//     XCD-aware tile order.

#include "bfp8_device.hpp"
#include "bfp8_launch.hpp"
#include "stream_common.hpp"

namespace bfp8 {

// ===================================================================== plan
StreamPlan plan_stream(int64_t M, int64_t N, int64_t K) {
    StreamPlan p;
    p.n_tiles = N / kStreamRows;
    p.m_tiles = (M + 15) / 16;
    const int64_t KB = K / 128;
    // Enough workgroups to give each of the 256 CUs one, but keep at least
    // one 128-K block per wave of a workgroup.
    const int64_t tiles = p.n_tiles * p.m_tiles;
    int64_t splits = 1;
    while (tiles * splits < 256 && KB / (splits * 2) >= kStreamWaves) splits *= 2;
    p.splits = splits;
    p.kb_per_split = (KB + splits - 1) / splits;
    return p;
}

size_t stream_workspace_bytes(const StreamPlan& p) {
    if (p.splits == 1) return 0;
    const size_t tiles = (size_t)(p.n_tiles * p.m_tiles);
    return stream_counter_bytes(p) + tiles * (size_t)p.splits * 256 * sizeof(float);
}

// =================================================================== stream
constexpr int kW8A8Chunk = 4;   // 128-K blocks per wave with loads in flight together

__global__ __launch_bounds__(kStreamThreads) void w8a8_stream_kernel(
    const uint8_t* __restrict__ xq, const float* __restrict__ xs,
    const uint8_t* __restrict__ wq, const float* __restrict__ ws,
    void* __restrict__ y, int y_dtype, int64_t M, int64_t N, int64_t K,
    int64_t n_tiles, int64_t splits, int64_t kb_per_split,
    float* __restrict__ partials, uint32_t* __restrict__ counters) {
    __shared__ float red[kStreamWaves * 256];
    const int64_t nt = blockIdx.x, split = blockIdx.y, mt = blockIdx.z;
    const int64_t KB = K / 128;
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const int r = lane & 15, g = lane >> 4;

    const int64_t n = nt * 16 + r;                 // weight row supplied by this lane
    const int64_t m = mt * 16 + r;                 // token supplied by this lane (and its output column)
    const bool m_ok = m < M;
    const int64_t kb_begin = split * kb_per_split;
    const int64_t kb_end = kb_begin + kb_per_split < KB ? kb_begin + kb_per_split : KB;

    const uint8_t* wrow = wq + n * K + g * 32;
    const uint8_t* xrow = xq + (m_ok ? m : 0) * K + g * 32;
    const float* ws_row = ws + (nt * 16 / 128) * KB;
    const float* xs_row = xs + (m_ok ? m : 0) * KB;

    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
    const f32x4 zero = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int64_t kb0 = kb_begin + wave; kb0 < kb_end; kb0 += kStreamWaves * kW8A8Chunk) {
        u32x4 wa[kW8A8Chunk][2], xb[kW8A8Chunk][2];
        float sc[kW8A8Chunk];
#pragma unroll
        for (int c = 0; c < kW8A8Chunk; ++c) {
            const int64_t kb = kb0 + c * kStreamWaves;
            if (kb < kb_end) {
                wa[c][0] = load_nt_16B(wrow + kb * 128);
                wa[c][1] = load_nt_16B(wrow + kb * 128 + 16);
            }
        }
#pragma unroll
        for (int c = 0; c < kW8A8Chunk; ++c) {
            const int64_t kb = kb0 + c * kStreamWaves;
            if (kb < kb_end) {
                if (m_ok) {
                    xb[c][0] = load_16B(xrow + kb * 128);
                    xb[c][1] = load_16B(xrow + kb * 128 + 16);
                    sc[c] = xs_row[kb] * ws_row[kb];
                } else {
                    xb[c][0] = xb[c][1] = u32x4{0u, 0u, 0u, 0u};
                    sc[c] = 0.0f;
                }
            }
        }
#pragma unroll
        for (int c = 0; c < kW8A8Chunk; ++c) {
            const int64_t kb = kb0 + c * kStreamWaves;
            if (kb < kb_end) {
                const i32x8 a = __builtin_bit_cast(i32x8, __builtin_shufflevector(wa[c][0], wa[c][1], 0, 1, 2, 3, 4, 5, 6, 7));
                const i32x8 b = __builtin_bit_cast(i32x8, __builtin_shufflevector(xb[c][0], xb[c][1], 0, 1, 2, 3, 4, 5, 6, 7));
                const f32x4 blk = mfma_e4m3_16x16x128(a, b, zero);
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[i] = __builtin_fmaf(blk[i], sc[c], acc[i]);
            }
        }
    }
    stream_finish(acc, red, y, y_dtype, M, N, nt, mt, splits, split, n_tiles, partials, counters);
}

hipError_t launch_w8a8_stream(const uint8_t* xq, const float* xs, const uint8_t* wq, const float* ws,
                              void* y, int y_dtype, int64_t M, int64_t N, int64_t K,
                              void* workspace, hipStream_t stream) {
    const StreamPlan p = plan_stream(M, N, K);
    uint32_t* counters;
    float* partials;
    stream_workspace_parts(p, workspace, counters, partials);
    hipLaunchKernelGGL(w8a8_stream_kernel, dim3((unsigned)p.n_tiles, (unsigned)p.splits, (unsigned)p.m_tiles),
                       dim3(kStreamThreads), 0, stream, xq, xs, wq, ws, y, y_dtype, M, N, K,
                       p.n_tiles, p.splits, p.kb_per_split, partials, counters);
    return hipGetLastError();
}

// ===================================================================== tile
constexpr int kTileN = 128;             // weight rows per workgroup
constexpr int kTileM = 128;             // tokens per workgroup
constexpr int kTileK = 128;             // one scale block per stage
constexpr int kTileThreads = 256;       // 4 waves, 2 (n) x 2 (m), 64x64 each
constexpr int kLdsRow = kTileK + 16;    // padded LDS row, bytes (keeps 16-byte alignment)
constexpr int kLdsStage = (kTileN + kTileM) * kLdsRow;

__device__ __forceinline__ void tile_coords(int64_t bid, int64_t tiles_n, int64_t tiles_m,
                                            int64_t& tn, int64_t& tm) {
    const int64_t total = tiles_n * tiles_m;
    // Workgroups are dealt round-robin to the 8 XCDs; give each XCD a
    // contiguous run of tiles so that the tiles sharing A or B rows share
    // that XCD's L2.
    int64_t t = bid;
    if (total % 8 == 0) t = (bid % 8) * (total / 8) + bid / 8;
    // Grouped order: walk 8 token tiles down before moving to the next weight tile.
    constexpr int64_t kGroup = 8;
    const int64_t per_group = kGroup * tiles_n;
    const int64_t group = t / per_group;
    const int64_t first_m = group * kGroup;
    const int64_t group_m = tiles_m - first_m < kGroup ? tiles_m - first_m : kGroup;
    const int64_t in_group = t - group * per_group;
    tm = first_m + in_group % group_m;
    tn = in_group / group_m;
}

__global__ __launch_bounds__(kTileThreads) void w8a8_tile_kernel(
    const uint8_t* __restrict__ xq, const float* __restrict__ xs,
    const uint8_t* __restrict__ wq, const float* __restrict__ ws,
    void* __restrict__ y, int y_dtype, int64_t M, int64_t N, int64_t K,
    int64_t tiles_n, int64_t tiles_m) {
    __shared__ __attribute__((aligned(16))) uint8_t lds[2 * kLdsStage];
    int64_t tn, tm;
    tile_coords(blockIdx.x, tiles_n, tiles_m, tn, tm);
    const int64_t n0 = tn * kTileN, m0 = tm * kTileM;
    const int64_t KB = K / 128;
    const int t = threadIdx.x;
    const int wave = t / kWave, lane = t % kWave;
    const int wn = wave & 1, wm = wave >> 1;
    const int r = lane & 15, g = lane >> 4;

    // Global -> LDS copy: thread t moves 16 bytes of rows (t / 8) + 32 i of
    // both the weight tile and the token tile.
    const int cp_row = t >> 3, cp_col = (t & 7) * 16;
    const uint8_t* a_src[4];
    const uint8_t* b_src[4];
    bool a_ok[4], b_ok[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t nrow = n0 + cp_row + 32 * i, mrow = m0 + cp_row + 32 * i;
        a_ok[i] = nrow < N;
        b_ok[i] = mrow < M;
        a_src[i] = wq + (a_ok[i] ? nrow : 0) * K + cp_col;
        b_src[i] = xq + (b_ok[i] ? mrow : 0) * K + cp_col;
    }
    u32x4 ra[4], rb[4];
    auto fetch = [&](int64_t kb) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            ra[i] = a_ok[i] ? load_16B(a_src[i] + kb * 128) : u32x4{0u, 0u, 0u, 0u};
            rb[i] = b_ok[i] ? load_16B(b_src[i] + kb * 128) : u32x4{0u, 0u, 0u, 0u};
        }
    };
    auto stash = [&](int buf) {
        uint8_t* base = lds + buf * kLdsStage;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            *reinterpret_cast<u32x4*>(base + (cp_row + 32 * i) * kLdsRow + cp_col) = ra[i];
            *reinterpret_cast<u32x4*>(base + (kTileN + cp_row + 32 * i) * kLdsRow + cp_col) = rb[i];
        }
    };

    // Token scales: lane's token for sub-tile j is m0 + 64 wm + 16 j + r.
    const float* xs_ptr[4];
    bool xs_ok[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int64_t mm = m0 + 64 * wm + 16 * j + r;
        xs_ok[j] = mm < M;
        xs_ptr[j] = xs + (xs_ok[j] ? mm : 0) * KB;
    }
    const float* ws_row = ws + tn * KB;   // kTileN == 128: one weight-scale row per tile

    f32x4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    const f32x4 zero = {0.0f, 0.0f, 0.0f, 0.0f};

    fetch(0);
    stash(0);
    __syncthreads();
    for (int64_t kb = 0; kb < KB; ++kb) {
        const int buf = (int)(kb & 1);
        if (kb + 1 < KB) fetch(kb + 1);
        float sc[4];
        const float wsc = ws_row[kb];
#pragma unroll
        for (int j = 0; j < 4; ++j) sc[j] = xs_ok[j] ? xs_ptr[j][kb] * wsc : 0.0f;

        const uint8_t* base = lds + buf * kLdsStage;
        i32x8 af[4], bf[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint8_t* p = base + (64 * wn + 16 * i + r) * kLdsRow + 32 * g;
            af[i] = __builtin_bit_cast(i32x8, __builtin_shufflevector(*reinterpret_cast<const u32x4*>(p),
                                                                      *reinterpret_cast<const u32x4*>(p + 16),
                                                                      0, 1, 2, 3, 4, 5, 6, 7));
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint8_t* p = base + (kTileN + 64 * wm + 16 * j + r) * kLdsRow + 32 * g;
            bf[j] = __builtin_bit_cast(i32x8, __builtin_shufflevector(*reinterpret_cast<const u32x4*>(p),
                                                                      *reinterpret_cast<const u32x4*>(p + 16),
                                                                      0, 1, 2, 3, 4, 5, 6, 7));
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const f32x4 blk = mfma_e4m3_16x16x128(af[i], bf[j], zero);
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[i][j][e] = __builtin_fmaf(blk[e], sc[j], acc[i][j][e]);
            }
        }
        if (kb + 1 < KB) stash(buf ^ 1);
        __syncthreads();
    }

    // Epilogue: lane holds n = n0 + 64 wn + 16 i + 4 g + e (e = 0..3) of token m.
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int64_t mm = m0 + 64 * wm + 16 * j + r;
        if (mm >= M) continue;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t nn = n0 + 64 * wn + 16 * i + 4 * g;
            if (nn >= N) continue;
            const f32x4 v = acc[i][j];
            if (y_dtype == 2) {
                *reinterpret_cast<f32x4*>(static_cast<float*>(y) + mm * N + nn) = v;
            } else {
                uint32_t h[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) h[e] = y_dtype == 0 ? float_to_bf16_bits(v[e]) : float_to_f16_bits(v[e]);
                *reinterpret_cast<uint2*>(static_cast<uint16_t*>(y) + mm * N + nn) =
                    make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
            }
        }
    }
}

hipError_t launch_w8a8_tile(const uint8_t* xq, const float* xs, const uint8_t* wq, const float* ws,
                            void* y, int y_dtype, int64_t M, int64_t N, int64_t K, hipStream_t stream) {
    const int64_t tiles_n = (N + kTileN - 1) / kTileN, tiles_m = (M + kTileM - 1) / kTileM;
    hipLaunchKernelGGL(w8a8_tile_kernel, dim3((unsigned)(tiles_n * tiles_m)), dim3(kTileThreads), 0, stream,
                       xq, xs, wq, ws, y, y_dtype, M, N, K, tiles_n, tiles_m);
    return hipGetLastError();
}

}  // namespace bfp8
