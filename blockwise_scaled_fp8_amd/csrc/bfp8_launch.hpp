// Internal launch functions of libbfp8: one per kernel family.  They assume
// arguments already validated by the C entry points and only enqueue work.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace bfp8 {

// Largest M that the W8A8 codes path always serves with the weight-streaming
// kernel.
#ifndef BFP8_STREAM_MAX_M
#define BFP8_STREAM_MAX_M 16
#endif
constexpr int64_t kStreamMaxM = BFP8_STREAM_MAX_M;
// W8A8 dispatch (codes in), from the projection sweep: the streaming kernel
// for M <= 16, and with two 16-token tiles per workgroup for M <= 32 on
// projections of at most 2^24 weights (4096 x 4096: 10.5 vs 12.2 us tiled;
// 1024 x 4096: 8.4 vs 9.8 us), the tiled kernels otherwise (12288 x 4096 at
// M = 32: 22.4 us tiled vs 28.2 us streamed).
inline bool w8a8_streams(int64_t M, int64_t N, int64_t K) {
    return M <= kStreamMaxM || (M <= 2 * kStreamMaxM && N * K <= ((int64_t)1 << 24));
}
// Rows of W covered by one streaming workgroup (one MFMA row tile).
constexpr int64_t kStreamRows = 16;
// Largest K of every GEMM: the tiled kernels address 256 rows x K bytes and
// the streaming kernels 16 rows x K bytes through 32-bit buffer offsets.
constexpr int64_t kTileMaxK = (int64_t)1 << 23;
// Workspace bytes of the tiled W8A8 kernels (split-K partial tiles and tile
// counters; 0 when the shape is not split).
size_t tile_workspace_bytes(int64_t M, int64_t N, int64_t K);
// Workspace bytes of the tiled W8A16 kernels.
size_t tile16_workspace_bytes(int64_t M, int64_t N, int64_t K);

// Split-K plan of a streaming kernel: a workgroup covers 16 weight rows and
// `mt_per_wg` 16-token tiles; `splits` workgroups share one such block of
// output tiles, each covering `kb_per_split` 128-K blocks.  Counters and
// partial tiles are kept per 16x16 output tile.
struct StreamPlan {
    int64_t n_tiles, m_tiles, mt_per_wg, splits, kb_per_split;
};
StreamPlan plan_stream(int64_t M, int64_t N, int64_t K, int64_t mt_per_wg = 1);
// The W8A8 codes kernel's plan: 1 or 2 token tiles per workgroup by M.
StreamPlan plan_stream_w8a8(int64_t M, int64_t N, int64_t K);
// Workspace bytes of a streaming plan: tile counters, then fp32 partial tiles.
size_t stream_workspace_bytes(const StreamPlan& p);

hipError_t launch_quant_act_1x128(const void* x, bool bf16, int64_t M, int64_t K,
                                  uint8_t* xq, float* xs, hipStream_t stream);
hipError_t launch_quant_weight_128x128(const void* w, bool bf16, int64_t N, int64_t K,
                                       uint8_t* wq, float* ws, hipStream_t stream);
hipError_t launch_dequant_weight(const uint8_t* wq, const float* scales, int block, void* w, int w_dtype,
                                 int64_t N, int64_t K, hipStream_t stream);

hipError_t launch_w8a8_tile(const uint8_t* xq, const float* xs, const uint8_t* wq, const float* ws,
                            void* y, int y_dtype, int64_t M, int64_t N, int64_t K, void* workspace,
                            hipStream_t stream);
hipError_t launch_w8a8_stream(const uint8_t* xq, const float* xs, const uint8_t* wq, const float* ws,
                              void* y, int y_dtype, int64_t M, int64_t N, int64_t K,
                              void* workspace, hipStream_t stream);
// Largest M for which the W8A8 streaming kernel quantises its 16-bit
// activations itself; above it the fused call runs the quantiser first.
constexpr int64_t kFusedQuantMaxM = 8;
// Streaming W8A8 that quantises its 16-bit activations itself (M <= kFusedQuantMaxM).
hipError_t launch_w8a8_stream_quant(const void* x, bool x_bf16, const uint8_t* wq, const float* ws,
                                    void* y, int y_dtype, int64_t M, int64_t N, int64_t K,
                                    void* workspace, hipStream_t stream);
hipError_t launch_w8a16_tile(const void* x, bool x_bf16, const uint8_t* wq, const float* ws, void* y,
                             int y_dtype, int64_t M, int64_t N, int64_t K, void* workspace, hipStream_t stream);
hipError_t launch_w8a16_blk128_stream(const void* x, bool x_bf16, const uint8_t* wq, const float* ws,
                                      void* y, int y_dtype, int64_t M, int64_t N, int64_t K,
                                      void* workspace, hipStream_t stream);
hipError_t launch_w8a16_blk32_stream(const void* x, const uint8_t* wq, const uint8_t* e8m0,
                                     void* y, int y_dtype, int64_t M, int64_t N, int64_t K,
                                     void* workspace, hipStream_t stream);

}  // namespace bfp8
