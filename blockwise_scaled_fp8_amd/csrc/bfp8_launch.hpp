// Internal launch functions of libbfp8: one per kernel family.  They assume
// arguments already validated by the C entry points and only enqueue work.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace bfp8 {

// Largest M that the W8A8 codes path always serves with the weight-streaming
// kernel.
constexpr int64_t kStreamMaxM = 16;   // one 16-token MFMA column tile
// Largest K of every GEMM: the tiled kernels address 256 rows x K bytes and
// the streaming kernels 16 rows x K bytes through 32-bit buffer offsets.
constexpr int64_t kTileMaxK = (int64_t)1 << 23;
// Rows of W covered by one streaming workgroup (one MFMA row tile).
constexpr int64_t kStreamRows = 16;
// Workspace bytes of the tiled W8A8 kernels (split-K partial tiles and tile
// counters; 0 when the shape is not split).
size_t tile_workspace_bytes(int64_t M, int64_t N, int64_t K);
// Workspace bytes of the tiled W8A16 kernels.
size_t tile16_workspace_bytes(int64_t M, int64_t N, int64_t K);
// Leading bytes of the tiled W8A8 workspace that hold the zero-initialised
// tile counters (0 when the plan does not split K).
size_t tile_counter_bytes(int64_t M, int64_t N, int64_t K);
// The tiled kernels' choice for a shape (the same planner the launches use):
// workgroup tile (weight rows x tokens), waves, tiles and K splits.
struct TileInfo {
    int tile_n, tile_m, waves;
    int64_t tiles, splits;
};
TileInfo tile_info(int64_t M, int64_t N, int64_t K);     // W8A8 codes
TileInfo tile16_info(int64_t M, int64_t N, int64_t K);   // W8A16 (16-bit tokens)

// Split-K plan of a streaming kernel: a workgroup covers 16 weight rows and
// one 16-token tile; `splits` workgroups share one output tile, each
// covering `kb_per_split` 128-K blocks.  Counters and partial tiles are kept
// per 16x16 output tile.
struct StreamPlan {
    int64_t n_tiles, m_tiles, splits, kb_per_split;
};
StreamPlan plan_stream(int64_t M, int64_t N, int64_t K);

// Shape of a launch of the all-token kernels: kr 16-row weight tiles and
// kt 16-token tiles per workgroup, groups_n x groups_m workgroups.
struct WideShape {
    int kr, kt;
    unsigned groups_n, groups_m;
    int splits = 1;   // K parts over grid.z (W8A8 at long K), partial tiles handed off
};

// One-round choice of the W8A8 and W8A16 blk128 all-token shapes: when some
// candidate's launch fits one round on the CUs (at most 256 workgroups), the
// one with the most workgroups, the larger kr on a tie; otherwise the one
// with the fewest, the larger kr on a tie.  Two rounds of these kernels cost
// more than one round of larger tiles, and at equal counts more weight rows
// per workgroup cut the token bytes per output.
struct WidePick {
    WideShape best{1, 2, 0, 0};
    int64_t best_wg = -1;
    bool best_one_round = false;
    void consider(int kr, int kt, int64_t M, int64_t N) {
        if (kr > 1 && N <= 8 * kr) return;   // half the rows or more would be padding
        const int64_t gn = (N + 16 * kr - 1) / (16 * kr), gm = (M + 16 * kt - 1) / (16 * kt);
        const int64_t wg = gn * gm;
        const bool one_round = wg <= 256;
        const bool tie_kr = wg == best_wg && kr > best.kr;
        const bool better = best_wg < 0 || (one_round && !best_one_round) ||
                            (one_round && best_one_round && (wg > best_wg || tie_kr)) ||
                            (!one_round && !best_one_round && (wg < best_wg || tie_kr));
        if (better) {
            best = WideShape{kr, kt, (unsigned)gn, (unsigned)(gm > 65535 ? 65536 : gm)};
            best_wg = wg;
            best_one_round = one_round;
        }
    }
};

// W8A8: (kr, kt) with kr in {1, 2, 4}, kt = 1 for M <= 16 (one token tile:
// two would double the token loads and MFMAs for nothing; 1024 x 12288 M = 8
// 9.0 against 10.5 us, 2048 x 12288 M = 5 9.2 against 10.9, 12288 x 4096
// M = 16 11.5 against 12.0, 8192 x 4096 M = 16 8.7 against 9.1) and
// kt in {2, 4} above (kt = 4 only when M needs at least four token tiles),
// chosen by WidePick.  Measured (us, 32 rotated weight
// copies, K = 4096; the pick first): 4096 x 4096 M = 64 (2, 2) 8.4 against
// 10.7 for (4, 2), M = 96 (2, 4) 10.1 against 10.7 for (4, 2), M = 128
// (4, 2) 10.7 against 11.2 for (2, 4) and 14.2 for (4, 4), M = 160 / 192 /
// 256 (4, 4) 13.0 / 13.9 / 14.0 (192 / 192 / 256 workgroups) against 17.8
// for (2, 4) at M = 192; 1024 x 4096 M = 256 (2, 2) 5.9 against 6.8 for
// (1, 4), M = 512 (4, 2) 8.35 against 8.46 for (2, 4), M = 768 / 1024
// (4, 4) 10.2 / 11.6; 2048 x 4096 M = 128 (2, 2) 6.7 against 8.0 for (1, 4),
// M = 512 (4, 4) 12.7; 12288 x 4096 M = 32 (4, 2) 13.8 against 16.4 for
// (2, 2), M = 64 (4, 4) 17.1 against 21.9 for (2, 2); 16384 x 4096 M = 32
// (4, 2) 16.7 against 18.1.
//
// At K >= 12288, where the unsplit pick leaves three quarters of the CUs
// idle (at most 64 workgroups), the K blocks may also be split over two or
// four workgroups (grid.z; at least 24 blocks each), the last one of a tile
// summing the parts in split order: among the one-round configurations with
// more workgroups than the unsplit pick, the one with the most, then the
// largest tile (kr kt), then the larger kr.  Measured (us): 1024 x 12288
// M = 8 / 16 (1, 1) split 4 7.5 / 7.7 against 9.0 / 10.8 unsplit (64
// workgroups); with 128 unsplit workgroups no gain (2048 x 12288 M = 5
// (2, 1) split 4 9.36 against 9.2).  Where the unsplit pick already fills the CUs a
// split buys only a larger tile, and the hand-off of partial tiles cost
// what the larger tile saved (4096 x 12288, split against unsplit or
// tiled: M = 16 (4, 1) split 4 13.5 against 13.2 streamed, M = 32 (4, 2)
// split 4 16.3 against 16.8 for (1, 2), M = 64 (4, 4) split 4 21.2
// against 18.2 tiled, M = 128 (4, 4) split 2 25.0 against 25.0 tiled).
inline WideShape w8a8_wide_shape(int64_t M, int64_t N, int64_t K) {
    const int64_t m_tiles = (M + 15) / 16;
    WidePick pick;
    const int kt_lo = M <= 16 ? 1 : 2, kt_hi = M <= 16 ? 1 : 4;
    for (int kt = kt_lo; kt <= kt_hi; kt *= 2) {
        if (kt > 2 && kt > m_tiles) continue;
        for (int kr = 4; kr >= 1; kr /= 2) pick.consider(kr, kt, M, N);
    }
    WideShape best = pick.best;
    const int64_t unsplit_wg = (int64_t)best.groups_n * best.groups_m;
    int64_t best_wg = unsplit_wg;
    const int64_t KB = K / 128;
    // Long K, one 32-token group on 16-row weight tiles: every workgroup
    // reads all 32 token rows over K, twice its weight bytes.  Two-tile rows
    // with K split two ways keep the workgroup count and halve those reads
    // (4096x12288, M = 32: 17.2 -> 15.1 us).
    if (KB >= 96 && M > 16 && unsplit_wg > 64 && best.kr == 1 && best.kt == 2) {
        const int64_t gn = (N + 31) / 32, gm = (M + 31) / 32;
        if (gn * gm * 2 >= unsplit_wg && gn * gm * 2 <= 256) return WideShape{2, 2, (unsigned)gn, (unsigned)gm, 2};
    }
    if (KB < 96 || unsplit_wg > 64) return best;
    for (int kt = kt_lo; kt <= kt_hi; kt *= 2) {
        if (kt > 2 && kt > m_tiles) continue;
        for (int kr = 4; kr >= 1; kr /= 2) {
            if (kr > 1 && N <= 8 * kr) continue;
            for (int sp = 2; sp <= 4; sp *= 2) {
                if (KB / sp < 24) continue;
                const int64_t gn = (N + 16 * kr - 1) / (16 * kr), gm = (M + 16 * kt - 1) / (16 * kt);
                const int64_t wg = gn * gm * sp;
                if (wg > 256 || wg <= unsplit_wg || gm > 65535) continue;
                const int area = kr * kt, best_area = best.kr * best.kt;
                const bool better = wg > best_wg || (best.splits > 1 && wg == best_wg && area > best_area) ||
                                    (best.splits > 1 && wg == best_wg && area == best_area && kr > best.kr);
                if (better) {
                    best = WideShape{kr, kt, (unsigned)gn, (unsigned)gm, sp};
                    best_wg = wg;
                }
            }
        }
    }
    return best;
}
inline bool w8a8_wide_one_round(int64_t M, int64_t N, int64_t K) {
    const WideShape w = w8a8_wide_shape(M, N, K);
    return (int64_t)w.groups_n * w.groups_m * w.splits <= 256;
}
// Workspace of a W8A8 all-token launch: the split tiles' arrival counters
// (256-byte aligned), then each tile's fp32 partial tiles, split by split
// (kr kt output tiles of 64 lanes x 4 floats each); nothing when K is not
// split.
inline size_t w8a8_wide_counter_bytes(const WideShape& w) {
    if (w.splits == 1) return 0;
    return ((size_t)w.groups_n * w.groups_m * 4 + 255) / 256 * 256;
}
inline size_t w8a8_wide_workspace_bytes(const WideShape& w) {
    if (w.splits == 1) return 0;
    return w8a8_wide_counter_bytes(w) +
           (size_t)w.groups_n * w.groups_m * w.splits * (size_t)(w.kr * w.kt) * 256 * sizeof(float);
}

// W8A16 blk128: one 16-token tile (kt = 1) for M <= 16, else kt = 2 or 4
// (4 only when M needs at least four token tiles); kr = 1, 2 or 4, without
// (4, 4) (its slots do not fit LDS twice per wave) and (2, 4) (its token
// tiles go to different waves, each loading the same weight rows); chosen
// by WidePick.  Measured (us, K = 4096, 32 rotated weight copies; the pick
// first): 4096 x 4096 M = 16 (1, 1) 6.8 against 10.2 for (4, 1), M = 96
// (4, 2) 12.1 (192 workgroups) against 15.2 for (2, 4) (256), M = 128
// (4, 2) 12.1 against 16.4 for (2, 4); 12288 x 4096 M = 12 / 16 (4, 1)
// 12.7 / 13.1 against 15.0 / 15.4 for (2, 1), M = 24 / 32 (4, 2) 14.5 /
// 15.2 against 18.2 / 19.2 for (2, 2); 8192 x 4096 M = 16 (2, 1) 9.5
// against 11.4 for (4, 1), M = 32 (2, 2) 11.6 against 13.7 for (4, 2);
// 16384 x 4096 M = 16 (4, 1) 16.1 against 17.2 for (2, 1); 1024 x 4096
// M = 256 (2, 2) 7.7 against 9.4 for (4, 2), M = 512 (4, 2) 10.3 (the tiled
// kernel 19.1); 4096 x 7168 M = 32 (1, 2) 12.2 against 19.8 for (4, 2).
inline WideShape w16_wide_shape(int64_t M, int64_t N) {
    WidePick pick;
    if (M <= 16) {
        for (int kr = 4; kr >= 1; kr /= 2) pick.consider(kr, 1, M, N);
        return pick.best;
    }
    const int64_t m_tiles = (M + 15) / 16;
    for (int kt = 2; kt <= 4; kt += 2) {
        if (kt > 2 && kt > m_tiles) continue;
        for (int kr = 4; kr >= 1; kr /= 2)
            if (kt == 2 || kr == 1) pick.consider(kr, kt, M, N);
    }
    return pick.best;
}

// Block-32 all-token shape (kr <= 2: a workgroup's rows share one 32-row
// band of UE8M0 scales): for M <= 16 one 16-token tile and kr = 1 or 2,
// the fewest workgroups that still give one per CU, two row tiles on a tie,
// else the most workgroups (measured at M = 16 on the blk128 kernel, kR = 1
// against 2, us: 4096 x 4096 6.91 / 7.73, 1024 x 4096 4.59 / 5.33,
// 4096 x 12288 14.57 / 18.22, but 12288 x 4096 17.63 / 15.39); above 16
// tokens (kr, kt) in {1, 2} x {2, 4} by the same rule (kt = 4 only when M
// needs at least four token tiles; 4096 x 7168 M = 32 (1, 2) 12.2, M = 64
// (2, 2) 16.5).
inline WideShape blk32_wide_shape(int64_t M, int64_t N) {
    const int64_t m_tiles = (M + 15) / 16;
    WideShape best{1, M <= 16 ? 1 : 2, 0, 0};
    int64_t best_wg = -1;
    bool best_full = false;
    for (int kt = M <= 16 ? 1 : 2; kt <= (M <= 16 ? 1 : 4); kt *= 2) {
        if (kt > 2 && kt > m_tiles) continue;
        for (int kr = 2; kr >= 1; --kr) {
            const int64_t gn = (N + 16 * kr - 1) / (16 * kr), gm = (M + 16 * kt - 1) / (16 * kt);
            const int64_t wg = gn * gm;
            const bool full = wg >= 256;
            const bool better = best_wg < 0 || (full && (!best_full || wg < best_wg)) || (!full && !best_full && wg > best_wg);
            if (better) {
                best = WideShape{kr, kt, (unsigned)gn, (unsigned)(gm > 65535 ? 65536 : gm)};
                best_wg = wg;
                best_full = full;
            }
        }
    }
    return best;
}

// Largest M for which the W8A8 streaming kernel quantises its 16-bit
// activations itself; above it the fused call runs the quantiser first.
constexpr int64_t kFusedQuantMaxM = 8;
// W8A8 dispatch (codes in), from the projection sweep:
//  * the streaming kernel for M <= 16 when it needs no split of K, or when
//    N < 1024, except for 4 < M <= 16 with K <= 4096 where its launch takes
//    more than one round (over 256 weight-row tiles) and the all-token
//    kernel's fits one, and for 8 < M <= 16 where it leaves CUs idle
//    (fewer than 256 weight-row tiles); and for M <= 64 when its workgroups
//    fit one round unsplit;
//  * the all-token kernel (launch_w8a8_wide: every token of a 32- or
//    64-token group per workgroup, no split) for the other M <= 32, and
//    when K <= 4096 and either M * N <= 2^19 or N >= 512 and its launch
//    fits one round (w8a8_wide_shape; up to M * N = 2^20: M <= 256 at
//    N = 4096, M <= 1024 at N = 1024); measured
//    (us, 32 rotated weight copies): 1024 x 4096 at
//    M = 1 / 16: 4.3 / 4.4 against 5.3 / 5.5 streamed with K split 4 ways;
//    at M = 32: 4096 x 4096 6.7, 1024 x 4096 4.9, 12288 x 4096 16.5,
//    4096 x 12288 17.1 against 11.6, 9.8, 22.5 and 17.8 tiled; 4096 x 4096
//    at M = 48 / 64 / 96 / 128: 7.8 / 8.7 / 10.8 / 12.5 against 12.1 /
//    12.7 / 13.5 / 14.3 tiled; 1024 x 4096 at M = 128 / 256 / 512: 5.4 /
//    6.4 / 9.4 against 11.2 / 11.9 / 12.9; with four weight-row tiles per
//    workgroup 4096 x 4096 at M = 160 / 192 / 256 13.0 / 13.9 / 14.0 against
//    16.2 / 16.4 / 17.7 tiled, 2048 x 4096 at M = 384 / 512 12.2 / 12.7
//    against 16.5 / 17.1, 1024 x 4096 at M = 768 / 1024 10.2 / 11.6 against
//    15.4 / 16.6, 12288 x 4096 at M = 64 17.1 against 17.4; but two rounds
//    lose (4096 x 4096 M = 320 / 384: 21.4 / 21.9 against 18.5 / 20.4 tiled,
//    12288 x 4096 M = 48 / 128 18.8 / 25.5 against 16.2 / 22.5), and with
//    K > 4096 and M > 32 the tiled kernels win or tie (4096 x 12288 M = 64
//    / 128: 19.9 / 26.1 against 18.3 / 24.7; 2048 x 8192 M = 256 22.3
//    against 18.2);
//  * the tiled kernels otherwise.
inline bool w8a8_streams(int64_t M, int64_t N, int64_t K) {
    if (M <= kStreamMaxM) {
        if (N < 1024 || K > kTileMaxK) return true;
        const StreamPlan p = plan_stream(M, N, K);
        if (p.splits > 1) return false;
        // One round of the all-token kernel against several of the streaming
        // kernel's 16-row workgroups (us, streaming against all-token, K =
        // 4096): 12288 x 4096 M = 5 / 8 / 16 14.2 / 14.3 / 15.3 against
        // 12.1 / 11.8 / 12.1, 8192 x 4096 M = 5 / 8 / 16 9.8 / 10.2 / 10.8
        // against 9.2 / 9.2 / 9.2, 6144 x 4096 M = 16 10.2 against 8.1,
        // 16384 x 4096 M = 16 19.6 against 15.9.  Not at M <= 4 (12288 x
        // 4096 M = 2 / 4: 11.3 / 11.4 against 12.1 / 11.7), nor where the
        // streaming launch fits one round (4096 x 4096 M = 8 / 16: 5.7 / 6.1
        // against 6.2 / 6.4), nor at K = 8192 (8192 x 8192 M = 8 / 16: 15.1 /
        // 17.0 against 18.1 / 18.3).
        const int64_t wg = p.n_tiles * p.m_tiles;
        if (M > 4 && K <= 4096 && wg > 256 && w8a8_wide_one_round(M, N, K)) return false;
        // Fewer streaming workgroups than CUs (N < 4096): the all-token
        // kernel with one token tile, as many workgroups but eight waves each
        // keeping three blocks in flight, is ahead at every M and K measured
        // (us, streaming against all-token): 1024 x 4096 M = 2 / 4 / 16 3.99 /
        // 4.07 / 4.64 against 3.69 / 3.72 / 3.98, 2048 x 4096 M = 2 / 16
        // 4.68 / 5.56 against 4.29 / 4.82, 3072 x 4096 M = 8 / 16 5.32 / 5.89
        // against 5.33 / 5.61, 1024 x 8192 M = 8 6.86 against 5.69, 2048 x
        // 7168 M = 16 8.35 against 7.48, 2048 x 2048 M = 16 3.82 against 3.23.
        // Taken only above kFusedQuantMaxM tokens: up to there the fused
        // quantise + W8A8 call quantises inside the streaming kernel, and it
        // must run the codes call's kernel to give the same bits.
        return !(M > kFusedQuantMaxM && wg < 256);
    }
    // More than one token tile (one workgroup per weight-row tile and token
    // tile, the weights read once per token tile): on small projections,
    // where every such workgroup fits in one round on the CUs without a
    // split of K (measured, us: 1024 x 4096, M = 32 / 64: 4.6 / 4.7 against
    // 4.9 / 7.3 for the all-token kernel; at 4096 x 4096, M = 32, 9.7 vs 7.5).
    if (M > 4 * kStreamMaxM || K > kTileMaxK) return false;
    const StreamPlan p = plan_stream(M, N, K);
    return p.splits == 1 && p.n_tiles * p.m_tiles <= 256;
}
inline bool w8a8_wide(int64_t M, int64_t N, int64_t K) {
    if (K > kTileMaxK || w8a8_streams(M, N, K)) return false;
    // Past M * N = 2^19 only for N >= 512: with four or fewer 64-row tiles
    // the workgroups that share a token group sit on different XCDs and each
    // fetches it (4096 tokens x 256 rows: 21.1 us against 16.8 tiled;
    // 2048 x 512 14.8 against 16.8).
    return M <= 2 * kStreamMaxM ||
           (K <= 4096 && (M * N <= ((int64_t)1 << 19) || (N >= 512 && w8a8_wide_one_round(M, N, K))));
}
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
// M >= 1, N a multiple of 16, K <= kTileMaxK; needs no workspace.
hipError_t launch_w8a8_wide(const uint8_t* xq, const float* xs, const uint8_t* wq, const float* ws,
                            void* y, int y_dtype, int64_t M, int64_t N, int64_t K, void* workspace,
                            hipStream_t stream);
hipError_t launch_w8a8_stream(const uint8_t* xq, const float* xs, const uint8_t* wq, const float* ws,
                              void* y, int y_dtype, int64_t M, int64_t N, int64_t K,
                              void* workspace, hipStream_t stream);
// Streaming W8A8 that quantises its 16-bit activations itself (M <= kFusedQuantMaxM).
hipError_t launch_w8a8_stream_quant(const void* x, bool x_bf16, const uint8_t* wq, const float* ws,
                                    void* y, int y_dtype, int64_t M, int64_t N, int64_t K,
                                    void* workspace, hipStream_t stream);
hipError_t launch_w8a16_tile(const void* x, bool x_bf16, const uint8_t* wq, const float* ws, void* y,
                             int y_dtype, int64_t M, int64_t N, int64_t K, void* workspace, hipStream_t stream);
// The W8A16 tiled kernel for block-32 weights (fp16 activations; N a
// multiple of 32, the plan and workspace of launch_w8a16_tile).
hipError_t launch_w8a16_blk32_tile(const void* x, const uint8_t* wq, const uint8_t* e8m0, void* y, int y_dtype,
                                   int64_t M, int64_t N, int64_t K, void* workspace, hipStream_t stream);
// W8A16 (blk128 and block-32) with 8 < M <= 16, when the streaming plan
// would not split K: the all-token kernel with one 16-token tile.  Its
// token rows arrive by direct-to-LDS loads of whole lines into per-wave
// rings, where the streaming kernel's sixteen live token rows per block
// stay register loads in the MFMA layout (half lines); measured at M = 16
// (us, streaming against all-token): blk128 4096 x 4096 7.33 / 6.91,
// 4096 x 7168 11.2 / 9.41, 4096 x 12288 17.7 / 14.57, 1024 x 4096 6.35 /
// 4.59, 12288 x 4096 16.34 / 15.39.  At M <= 8 the streaming kernel, whose
// token rows already come through LDS there, stays ahead (M = 8: 5.95 vs
// 6.3 us at 4096 x 4096).
inline bool w8a16_one_tile(int64_t M, int64_t N, int64_t K) {
    return M > kStreamMaxM / 2 && M <= kStreamMaxM && K <= kTileMaxK && plan_stream(M, N, K).splits == 1;
}
// The W8A16 blk128 / block-32 all-token launch of an M x N product fits one
// round of workgroups on the 256 CUs.
inline bool w16_one_round(int64_t M, int64_t N) {
    const WideShape w = w16_wide_shape(M, N);
    return (int64_t)w.groups_n * w.groups_m <= 256;
}
inline bool blk32_one_round(int64_t M, int64_t N) {
    const WideShape w = blk32_wide_shape(M, N);
    return (int64_t)w.groups_n * w.groups_m <= 256;
}
// W8A16 blk128 dispatch: the streaming kernel for M <= 16 except where
// w8a16_one_tile holds or, at 4 <= M <= 8, the streaming launch would take
// several rounds; the all-token kernel (launch_w8a16_wide) there, for
// M > 16 when K <= 4096 and either M <= 32 or its launch fits one round
// (w16_wide_shape), and for 16 < M <= 64 when 4096 < K <= 8192 and its
// launch fits one round; the tiled kernel otherwise.  Measured, us
// (all-token against tiled; before four-row tiles): K = 4096
// N = 4096 M = 32 / 64 / 128 9.6 / 11.9 / 17.8 against 13.7 / 14.2 / 20.4;
// N = 1024 M = 64 / 128 / 256 7.0 / 7.5 / 9.8 against 11.5 / 17.0 / 18.1;
// N = 12288 M = 32 22.3 vs 26.3, but from M = 64 there the tiled kernel wins
// (27.5 vs 33.5); 4096 x 7168 M = 17 / 32 / 48 / 64 11.5 / 13.5 / 14.8 /
// 16.6 against 13.9 / 14.4 / 15.6 / 16.8, 1024 x 8192 M = 17 / 64 10.0 /
// 11.3 against 13.0 / 13.7; but 12288 x 8192 (two rounds) M = 17 / 32 34.1
// / 38.5 against 31.9 / 33.0 and 4096 x 12288 M = 17 / 32 18.2 / 22.2
// against 17.3 / 17.6.  With four-row tiles one round reaches further:
// 1024 x 4096 M = 512 10.3 against 19.1 tiled, 12288 x 4096 M = 64 (two
// rounds, left tiled) 22.9 against 25.9.
inline bool w8a16_wide(int64_t M, int64_t N, int64_t K) {
    if (w8a16_one_tile(M, N, K)) return true;
    if (M <= kStreamMaxM) {
        // 4 <= M <= 8 where the streaming launch takes several rounds and a
        // one-round all-token shape exists (us, streaming against all-token
        // with one token tile): 12288 x 4096 M = 4 / 8 13.4 / 14.2 against
        // 12.1 / 12.0.  Not where the streaming launch fits one round or
        // fewer (4096 x 4096 M = 4 5.57 against 6.21; 1024 x 4096 M = 2 / 4 /
        // 8 3.68 / 3.80 / 4.10 against 4.27 / 4.29 / 4.41).
        if (M < 4 || K > 4096) return false;
        const StreamPlan p = plan_stream(M, N, K);
        return p.splits == 1 && p.n_tiles * p.m_tiles > 256 && w16_one_round(M, N);
    }
    if (K <= 4096) return M <= 2 * kStreamMaxM || w16_one_round(M, N);
    return K <= 8192 && M <= 4 * kStreamMaxM && w16_one_round(M, N);
}
// Block-32 dispatch: the one-token kernel for M = 1 (K <= kOneTokenRouteK);
// the tiled kernel where blk32_tile holds; the all-token kernel
// (launch_w8a16_blk32_wide) for the other M > 8 whose streaming plan would
// not split K, one 16-token tile up to M = 16 and token groups of 32 or 64
// above (blk32_wide_shape); the streaming kernels otherwise (M <= 8, and where K
// is split: w8a16_blk32_stream_lds_kernel up to M = 16, one 16-token tile
// per workgroup above).  Above M = 16 the streaming
// kernel runs one 16-token tile per workgroup and so reads the weights
// once per tile; measured at 4096 x 7168 (us, streaming against
// all-token): M = 17 19.8 / 11.4, 32 23.8 / 13.4, 64 44.0 / 16.5,
// 128 86.0 / 26.5, 256 170.2 / 43.3.
inline bool blk32_wide(int64_t M, int64_t N, int64_t K) {
    return M > kStreamMaxM / 2 && K <= kTileMaxK && plan_stream(M, N, K).splits == 1;
}
// Block-32 on the tiled MFMA kernel (launch_w8a16_blk32_tile, the W8A16
// tiles with the UE8M0 scales applied in the widening and no promotion
// step) for M > 16 whose streaming plan does not split K, unless the
// all-token kernel is ahead: K <= 4096 with M <= 32 or M <= 256 and
// M * N <= 2^19, or K <= 8192 with M <= 32 and a one-round launch.
// Measured (us, all-token / tiled): 4096 x 7168 M = 17 11.4 / 13.4,
// 32 13.4 / 13.7, 64 16.5 / 14.4, 128 26.7 / 21.4, 256 43.4 / 26.0,
// 512 76.9 / 38.1, 1024 145 / 63.2, 4096 548 / 204; 1024 x 4096 M = 64
// 6.3 / 9.9, 256 7.6 / 16.5, 1024 22.8 / 20.0; 12288 x 4096 M = 32 20.7 /
// 23.1, 64 31.4 / 23.1, 256 72.7 / 48.1; 4096 x 12288 M = 17 18.2 / 17.1;
// 2048 x 12288 M = 24 18.9 / 17.2.  Where the streaming plan splits K
// (few weight-row tiles, long K) the streaming kernel beats the tiled one:
// M = 20, 512 x 12288 8.2 vs 13.2; M = 17, 704 x 8320 9.2 vs 13.1; M = 32,
// 1024 x 16384 15.7 vs 20.4.
inline bool blk32_tile(int64_t M, int64_t N, int64_t K) {
    if (M <= kStreamMaxM || K > kTileMaxK || plan_stream(M, N, K).splits > 1) return false;
    if (K <= 4096) return !(M <= 2 * kStreamMaxM || (M <= 16 * kStreamMaxM && M * N <= ((int64_t)1 << 19)));
    return !(K <= 8192 && M <= 2 * kStreamMaxM && blk32_one_round(M, N));
}
// One token (W8A8 codes, W8A8 with activations quantised in the kernel,
// W8A16 blk128, block-32): dot-product kernels on the vector ALUs, no
// workspace (launch_w8a8_gemv, launch_w8a8_gemv_quant, launch_w8a16_gemv,
// launch_w8a16_blk32_gemv).  They are built for K up to kOneTokenMaxK and
// serve the K where they measured faster than the streaming MFMA kernels
// (us, at least 512 MB of rotated weight copies, after a clock ramp):
//   N = K = 4096: W8A8 codes 5.14, fused 4.96, W8A16 5.01 (streaming
//     kernels 5.45, 5.82, 5.69 when last compared);
//   4096 x 7168: W8A8 codes 7.10 vs 7.68, W8A16 7.11 vs 7.70, block-32
//     6.89 vs 7.65, fused 7.81 vs 7.66;
//   4096 x 12288: W8A16 10.67 vs 10.92, but W8A8 codes 12.19 vs 10.82 and
//     fused 14.17 vs 11.03.
// So W8A8 and block-32 take them up to K = 8192, W8A16 up to 12288.  The
// fused call keeps the codes call's range despite its 2 % loss at 7168: the
// two must run the same kernel to give the same bits.
constexpr int64_t kOneTokenMaxK = 16384;
constexpr int64_t kOneTokenRouteK = 8192;      // W8A8 (codes and fused), block-32
constexpr int64_t kOneTokenRouteK16 = 12288;   // W8A16 blk128
inline bool one_token(int64_t M, int64_t K) { return M == 1 && K <= kOneTokenRouteK; }
inline bool one_token_w8a16(int64_t M, int64_t K) { return M == 1 && K <= kOneTokenRouteK16; }
// The one-token kernels give each wave one weight row.  With four-wave
// workgroups that read the token from L2, two rows per wave paid on the
// largest projections (12288 x 4096: W8A8 10.6 vs 10.2 us); with eight-wave
// workgroups that share the token through LDS, one row is faster there too
// (W8A8 9.8 vs 10.6 us, W8A16 9.7 vs 10.55) and equal at 4096 x 7168.
constexpr int kGemvLaunchWaves = 8;    // waves per workgroup of the one-token kernels
constexpr int kStreamLaunchWaves = 16;  // waves per workgroup of the streaming kernels
// Waves per workgroup of the W8A8 all-token kernel for kr weight-row tiles
// and kt token tiles: four where a slot is large (kr = 4 or kt = 4), so
// that two or three slots per wave fit in LDS, else eight.
constexpr int w8a8_wide_waves(int kr, int kt) { return kr == 4 || kt == 4 ? 4 : 8; }
// W8A16 all-token kernel (kr weight-row tiles, kt token tiles): token tiles
// per wave, all of them wherever four waves' LDS rings hold them (every
// case but kt = 4 with kr = 2; kr = 4 only with kt <= 2), else one; and the
// waves per workgroup (four for kr = 4, whose weight slabs fill the slots).
constexpr int w16_wide_tiles_per_wave(int kr, int kt) { return kr == 4 ? kt : kt == 1 || (kt == 4 && kr == 2) ? 1 : kt; }
constexpr int w16_wide_waves(int kr, int kt) { return kr == 4 || w16_wide_tiles_per_wave(kr, kt) > 1 ? 4 : 8; }
constexpr int kQuantLaunchWaves = 4;    // waves per workgroup of the quantisers
// Workgroups of the 1x128 activation quantiser's grid.
int64_t quant_act_workgroups(int64_t M, int64_t K);
hipError_t launch_w8a8_gemv(const uint8_t* xq, const float* xs, const uint8_t* wq, const float* ws, void* y,
                            int y_dtype, int64_t N, int64_t K, hipStream_t stream);
hipError_t launch_w8a8_gemv_quant(const void* x, bool x_bf16, const uint8_t* wq, const float* ws, void* y,
                                  int y_dtype, int64_t N, int64_t K, hipStream_t stream);
hipError_t launch_w8a16_gemv(const void* x, bool x_bf16, const uint8_t* wq, const float* ws, void* y, int y_dtype,
                             int64_t N, int64_t K, hipStream_t stream);
// M >= 1, N a multiple of 16, K <= kTileMaxK; needs no workspace.
hipError_t launch_w8a16_wide(const void* x, bool x_bf16, const uint8_t* wq, const float* ws, void* y, int y_dtype,
                             int64_t M, int64_t N, int64_t K, hipStream_t stream);
hipError_t launch_w8a16_blk128_stream(const void* x, bool x_bf16, const uint8_t* wq, const float* ws,
                                      void* y, int y_dtype, int64_t M, int64_t N, int64_t K,
                                      void* workspace, hipStream_t stream);
// One token, block-32 weights (K <= kOneTokenMaxK, N a multiple of 32): dot products on the vector ALUs.
hipError_t launch_w8a16_blk32_gemv(const void* x, const uint8_t* wq, const uint8_t* e8m0, void* y, int y_dtype,
                                   int64_t N, int64_t K, hipStream_t stream);
hipError_t launch_w8a16_blk32_stream(const void* x, const uint8_t* wq, const uint8_t* e8m0,
                                     void* y, int y_dtype, int64_t M, int64_t N, int64_t K,
                                     void* workspace, hipStream_t stream);
// Block-32 all-token kernel (shape w16_wide_shape; N a multiple of 32, K of
// 128, K <= kTileMaxK); needs no workspace.
hipError_t launch_w8a16_blk32_wide(const void* x, const uint8_t* wq, const uint8_t* e8m0, void* y, int y_dtype,
                                   int64_t M, int64_t N, int64_t K, hipStream_t stream);

}  // namespace bfp8
