// Internal launch functions of libbfp8: one per kernel family.  They assume
// arguments already validated by the C entry points and only enqueue work.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace bfp8 {

// Largest M served by the weight-streaming (decode) kernel of W8A8.
#ifndef BFP8_STREAM_MAX_M
#define BFP8_STREAM_MAX_M 16
#endif
constexpr int64_t kStreamMaxM = BFP8_STREAM_MAX_M;
// Rows of W covered by one streaming workgroup (one MFMA row tile).
constexpr int64_t kStreamRows = 16;
// Largest K of every GEMM: the tiled kernels address 256 rows x K bytes and
// the streaming kernels 16 rows x K bytes through 32-bit buffer offsets.
constexpr int64_t kTileMaxK = (int64_t)1 << 23;
// Workspace bytes of the tiled W8A8 kernels (split-K partial tiles and tile
// counters; 0 when the shape is not split).
size_t tile_workspace_bytes(int64_t M, int64_t N, int64_t K);

// Split-K plan of a streaming kernel: `splits` workgroups share one
// (16-row, 16-token) output tile, each covering `kb_per_split` 128-K blocks.
struct StreamPlan {
    int64_t n_tiles, m_tiles, splits, kb_per_split;
};
StreamPlan plan_stream(int64_t M, int64_t N, int64_t K);
// Workspace bytes of a streaming plan: tile counters, then fp32 partial tiles.
size_t stream_workspace_bytes(const StreamPlan& p);

hipError_t launch_quant_act_1x128(const void* x, bool bf16, int64_t M, int64_t K,
                                  uint8_t* xq, float* xs, hipStream_t stream);
hipError_t launch_quant_weight_128x128(const void* w, bool bf16, int64_t N, int64_t K,
                                       uint8_t* wq, float* ws, hipStream_t stream);

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
hipError_t launch_w8a16_blk128_stream(const void* x, bool x_bf16, const uint8_t* wq, const float* ws,
                                      void* y, int y_dtype, int64_t M, int64_t N, int64_t K,
                                      void* workspace, hipStream_t stream);
hipError_t launch_w8a16_blk32_stream(const void* x, const uint8_t* wq, const uint8_t* e8m0,
                                     void* y, int y_dtype, int64_t M, int64_t N, int64_t K,
                                     void* workspace, hipStream_t stream);

}  // namespace bfp8
