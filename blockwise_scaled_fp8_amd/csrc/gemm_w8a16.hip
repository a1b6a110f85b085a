// W8A16 GEMMs for gfx950: 16-bit activations, E4M3 weights expanded to
// 16 bits in registers.
//
// There is no MFMA that multiplies a 16-bit operand by an FP8 operand, so
// with 16-bit activations the weights are widened to the activations' type
// and the bf16/fp16 MFMA runs ([3090] §2: mixed operand types do not exist
// in one matrix instruction).  The widening is exact and takes one gfx950
// conversion instruction per two weights (widen8); at decode sizes the
// kernels are bound by streaming the weights from HBM, and the widening
// hides under the loads ([3090] §4.3).
//
// blk128: weights with one fp32 scale per 128x128 tile, widened to their
// exact bf16 or fp16 values, so the per-block promotion is one FMA per
// output: acc += P * ws ([ARC] "What this adds").
//
// blk32 (UE8M0): weights with one power-of-two scale 2^e per 32x32 tile.
// The conversion applies 2^e itself: each weight becomes the fp16 number
// value * 2^e, exact for e in [-14, 7] ([SM70] "Exactness"), so the MFMA
// sees exactly the weights of a load-time fp16 dequantisation and
// accumulates in fp32 across all K.
//
// M = 1 with K <= 12288 (block-32: 8192) runs a plain dot-product kernel on
// the vector ALUs (w8a16_gemv_kernel, w8a16_blk32_gemv_kernel below).  The other kernels here stream the weights like
// the W8A8 decode kernel: one
// workgroup per 16 weight rows (and per split of K), 16 tokens on the MFMA
// column axis, sixteen waves taking interleaved 128-K blocks.  W8A16 blk128
// with M > 16 runs the tiled MFMA kernel instead (gemm_w8a8_tile.hip); blk32
// with M > 16 is served by more token tiles, each streaming the weights again.
//
// Operand mapping: within a 128-K block, lane l (row/column l % 16, slot
// g = l / 16) holds the 16-byte weight chunks g and g + 4 of its row (K
// offsets 16 g and 64 + 16 g).  MFMA j (j = 0..3) takes 8 of those 32
// values: K offsets 16 g + 8 j for j < 2 and 64 + 16 g + 8 (j - 2) for
// j >= 2; the activation operand of MFMA j is loaded with the same mapping,
// so the contraction covers each K index once.

#include "bfp8_device.hpp"
#include "bfp8_launch.hpp"
#include "stream_common.hpp"

namespace bfp8 {

constexpr int kW8A16Chunk = 4;   // 128-K blocks per wave with loads in flight together

// blk32 with M > 16: one 16-token tile per workgroup (grid z), register
// loads for weights and tokens.
__global__ __launch_bounds__(kStreamThreads) void w8a16_blk32_stream_kernel(
    const uint16_t* __restrict__ x, const uint8_t* __restrict__ wq, const uint8_t* __restrict__ e8m0,
    void* __restrict__ y, int y_dtype, int64_t M, int64_t N, int64_t K,
    int64_t n_tiles, int64_t splits, int64_t kb_per_split,
    float* __restrict__ partials, uint32_t* __restrict__ counters) {
    __shared__ float red[kStreamRedWords];
    const int64_t nt = blockIdx.x, split = blockIdx.y, mt = blockIdx.z;
    const int64_t KB = K / 128, K32 = K / 32;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave), lane = threadIdx.x % kWave;
    const int r = lane & 15, g = lane >> 4;
    const int64_t n = nt * 16 + r;
    const int64_t m = mt * 16 + r;
    const bool m_ok = m < M;
    const int64_t kb_begin = split * kb_per_split;
    const int64_t kb_end = kb_begin + kb_per_split < KB ? kb_begin + kb_per_split : KB;

    const uint8_t* wrow = wq + n * K + g * 16;
    const uint16_t* xrow = x + (m_ok ? m : 0) * K + g * 16;
    // This lane's chunk g of block kb lies in 32x32 tile (n / 32, 4 kb + g / 2)
    // and its chunk g + 4 in tile (n / 32, 4 kb + 2 + g / 2).
    const uint8_t* erow = e8m0 + (n / 32) * K32 + (g >> 1);

    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int64_t kb0 = kb_begin + wave; kb0 < kb_end; kb0 += kStreamWaves * kW8A16Chunk) {
        u32x4 wa[kW8A16Chunk][2], xb[kW8A16Chunk][4];
        uint32_t ebyte[kW8A16Chunk][2];
        // Activations and scale bytes first (from L2), then the weight stream;
        // every load is issued before any wait (rows past M: see above).
#pragma unroll
        for (int c = 0; c < kW8A16Chunk; ++c) {
            const int64_t kb = kb0 + c * kStreamWaves;
            if (kb < kb_end) {
#pragma unroll
                for (int j = 0; j < 4; ++j) xb[c][j] = load_16B(xrow + kb * 128 + (j < 2 ? 8 * j : 64 + 8 * (j - 2)));
                ebyte[c][0] = erow[kb * 4];
                ebyte[c][1] = erow[kb * 4 + 2];
            }
        }
#pragma unroll
        for (int c = 0; c < kW8A16Chunk; ++c) {
            const int64_t kb = kb0 + c * kStreamWaves;
            if (kb < kb_end) {
                wa[c][0] = load_16B(wrow + kb * 128);
                wa[c][1] = load_16B(wrow + kb * 128 + 64);
            }
        }
        asm volatile("" ::: "memory");   // compiler-only: all loads above before the first wait
#pragma unroll
        for (int c = 0; c < kW8A16Chunk; ++c) {
            const int64_t kb = kb0 + c * kStreamWaves;
            if (kb < kb_end) {
                // MFMAs 0, 1 take K offsets below 64 (the first 32x32 tile of the
                // block for this lane's slot), MFMAs 2, 3 the second.
                const float e0 = ue8m0_scale(ebyte[c][0]), e1 = ue8m0_scale(ebyte[c][1]);
                const uint32_t q[8] = {wa[c][0][0], wa[c][0][1], wa[c][0][2], wa[c][0][3],
                                       wa[c][1][0], wa[c][1][1], wa[c][1][2], wa[c][1][3]};
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const u32x4 a = widen8<false>(q[2 * j], q[2 * j + 1], j < 2 ? e0 : e1);
                    acc = mfma_f16_16x16x32(a, m_ok ? xb[c][j] : u32x4{0u, 0u, 0u, 0u}, acc);
                }
            }
        }
    }
    stream_finish(acc, red, y, y_dtype, M, N, nt, mt, splits, split, n_tiles, partials, counters);
}

// M <= 16 (padded token count Mp = 1, 2, 4, 8 or 16): the weights come
// through LDS slabs as whole 128-byte lines (two loads of eight full lines
// per block, where register loads in the MFMA layout read sixteen half
// lines), and for Mp <= 8 the block's token rows as direct-to-LDS dword
// loads (one per token row and block), all issued before the first wait.
// Per wave and block that is two weight loads and Mp token loads, where
// register token loads take four 16-byte loads per lane (sixteen lanes of
// one token column reading the same row when M = 1).  With Mp = 16 every
// lane carries a live token row, so the token loads stay register loads
// (and sixteen 256-byte rows per block would not fit beside the slabs).
// Lanes past the token count read row 0 and are zeroed by a select.
constexpr int kW8A16LdsMaxM = 16;
constexpr int kW8A16LdsChunk = 2;
static_assert(kW8A16LdsChunk == 2, "wait_block counts two blocks per pass");

template <bool kXBf16, int kMp>
__global__ __launch_bounds__(kStreamThreads) void w8a16_blk128_stream_lds_kernel(
    const uint16_t* __restrict__ x, const uint8_t* __restrict__ wq, const float* __restrict__ ws,
    void* __restrict__ y, int y_dtype, int64_t M, int64_t N, int64_t K,
    int64_t n_tiles, int64_t splits, int64_t kb_per_split,
    float* __restrict__ partials, uint32_t* __restrict__ counters) {
    constexpr bool kRegX = kMp == 16;   // sixteen live token rows: register loads, no LDS rows
    __shared__ __attribute__((aligned(16))) uint8_t xrows[kStreamWaves][kW8A16LdsChunk][kRegX ? 16 : kMp * kXRowStride];
    __shared__ __attribute__((aligned(1024))) uint8_t wslab[kStreamWaves][kW8A16LdsChunk][kSlabBytes];
    float* red = slab_scratch(&wslab[0][0][0]);   // used after the last block only
    const int64_t nt = blockIdx.x, split = blockIdx.y;
    const bool nt_loads = weights_nt(N, K);   // M <= 16: one token tile, no other workgroup reads these weights
    const int64_t KB = K / 128;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave), lane = threadIdx.x % kWave;
    const int r = lane & 15, g = lane >> 4;
    const bool r_ok = r < kMp && r < M;
    const int r_row = r < kMp ? r : 0;
    // Register path: lane (r, g) reads its K slices of token r straight
    // from memory (rows past M read row 0, zeroed by the select).
    const uint16_t* xreg = x + (r_ok ? r : 0) * K + g * 16;
    const int64_t kb_begin = split * kb_per_split;
    const int64_t kb_end = kb_begin + kb_per_split < KB ? kb_begin + kb_per_split : KB;

    const i32x4 rsrc_w = buffer_rsrc(wq + nt * 16 * K, (uint32_t)(16 * K));
    const i32x4 rsrc_x = buffer_rsrc(x, (uint32_t)(M * K * 2));
    const int lane_off_w = slab_lane_offset(lane, K);
    const float* ws_row = ws + (nt * 16 / 128) * KB;

    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
    const f32x4 zero = {0.0f, 0.0f, 0.0f, 0.0f};
    const u32x4 z4 = {0u, 0u, 0u, 0u};
    for (int64_t kb0 = kb_begin + wave; kb0 < kb_end; kb0 += kStreamWaves * kW8A16LdsChunk) {
        float wsv[kW8A16LdsChunk];
        u32x4 xr[kW8A16LdsChunk][4];
#pragma unroll
        for (int c = 0; c < kW8A16LdsChunk; ++c) {
            const int64_t kb = kb0 + c * kStreamWaves;
            if (kb < kb_end) {
                wsv[c] = ws_row[kb];
                if constexpr (kRegX) {
#pragma unroll
                    for (int j = 0; j < 4; ++j) xr[c][j] = load_16B(xreg + kb * 128 + (j < 2 ? 8 * j : 64 + 8 * (j - 2)));
                }
            }
        }
        if constexpr (!kRegX) {
#pragma unroll
            for (int c = 0; c < kW8A16LdsChunk; ++c) {
                const int64_t kb = kb0 + c * kStreamWaves;
                if (kb < kb_end) xrows_issue<kMp>(xrows[wave][c], rsrc_x, lane, K, kb);
            }
        }
#pragma unroll
        for (int c = 0; c < kW8A16LdsChunk; ++c) {
            const int64_t kb = kb0 + c * kStreamWaves;
            if (kb < kb_end) slab_issue(wslab[wave][c], rsrc_w, lane_off_w, K, kb, nt_loads);
        }
        const bool two = kb0 + kStreamWaves < kb_end;     // wave-uniform
#pragma unroll
        for (int c = 0; c < kW8A16LdsChunk; ++c) {
            const int64_t kb = kb0 + c * kStreamWaves;
            if (kb < kb_end) {
                wait_block(c, two);
                u32x4 wa0, wa1;
                slab_read(wslab[wave][c], r, g, wa0, wa1);
                const uint32_t q[8] = {wa0[0], wa0[1], wa0[2], wa0[3], wa1[0], wa1[1], wa1[2], wa1[3]};
                // MFMA j takes K offsets 16 g + 8 j (j < 2) and 64 + 16 g + 8 (j - 2):
                // bytes 32 g + 16 j and 128 + 32 g + 16 (j - 2) of the token row.
                const uint8_t* row = xrows[wave][c] + r_row * kXRowStride + 32 * g;
                u32x4 xv[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    if constexpr (kRegX) xv[j] = xr[c][j];
                    else xv[j] = *reinterpret_cast<const u32x4*>(row + (j < 2 ? 16 * j : 128 + 16 * (j - 2)));
                    xv[j] = r_ok ? xv[j] : z4;
                }
                f32x4 blk = zero;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const u32x4 a = widen8<kXBf16>(q[2 * j], q[2 * j + 1]);
                    blk = kXBf16 ? mfma_bf16_16x16x32(a, xv[j], blk) : mfma_f16_16x16x32(a, xv[j], blk);
                }
                const float sc = wsv[c];
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[i] = __builtin_fmaf(blk[i], sc, acc[i]);
            }
        }
    }
    __syncthreads();   // every wave is done with the slabs that red overlays
    stream_finish(acc, red, y, y_dtype, M, N, nt, 0, splits, split, n_tiles, partials, counters);
}

// blk32 for M <= 16, staged like w8a16_blk128_stream_lds_kernel: weight
// lines through LDS slabs, the block's fp16 token rows by direct-to-LDS
// loads for Mp <= 8 (register loads for Mp = 16), issued before the first
// wait; the scale bytes stay register loads.  The exact fp16 scaling and
// the accumulation across all K are those of w8a16_blk32_stream_kernel.
template <int kMp>
__global__ __launch_bounds__(kStreamThreads) void w8a16_blk32_stream_lds_kernel(
    const uint16_t* __restrict__ x, const uint8_t* __restrict__ wq, const uint8_t* __restrict__ e8m0,
    void* __restrict__ y, int y_dtype, int64_t M, int64_t N, int64_t K,
    int64_t n_tiles, int64_t splits, int64_t kb_per_split,
    float* __restrict__ partials, uint32_t* __restrict__ counters) {
    constexpr bool kRegX = kMp == 16;   // sixteen live token rows: register loads, no LDS rows
    __shared__ __attribute__((aligned(16))) uint8_t xrows[kStreamWaves][kW8A16LdsChunk][kRegX ? 16 : kMp * kXRowStride];
    __shared__ __attribute__((aligned(1024))) uint8_t wslab[kStreamWaves][kW8A16LdsChunk][kSlabBytes];
    float* red = slab_scratch(&wslab[0][0][0]);   // used after the last block only
    const int64_t nt = blockIdx.x, split = blockIdx.y;
    const bool nt_loads = weights_nt(N, K);   // M <= 16: one token tile, no other workgroup reads these weights
    const int64_t KB = K / 128, K32 = K / 32;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave), lane = threadIdx.x % kWave;
    const int r = lane & 15, g = lane >> 4;
    const bool r_ok = r < kMp && r < M;
    const int r_row = r < kMp ? r : 0;
    const uint16_t* xreg = x + (r_ok ? r : 0) * K + g * 16;
    const int64_t n = nt * 16 + r;
    const int64_t kb_begin = split * kb_per_split;
    const int64_t kb_end = kb_begin + kb_per_split < KB ? kb_begin + kb_per_split : KB;

    const i32x4 rsrc_w = buffer_rsrc(wq + nt * 16 * K, (uint32_t)(16 * K));
    const i32x4 rsrc_x = buffer_rsrc(x, (uint32_t)(M * K * 2));
    const int lane_off_w = slab_lane_offset(lane, K);
    // Chunk g of block kb lies in 32x32 tile (n / 32, 4 kb + g / 2), chunk
    // g + 4 in tile (n / 32, 4 kb + 2 + g / 2).
    const uint8_t* erow = e8m0 + (n / 32) * K32 + (g >> 1);

    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
    const u32x4 z4 = {0u, 0u, 0u, 0u};
    for (int64_t kb0 = kb_begin + wave; kb0 < kb_end; kb0 += kStreamWaves * kW8A16LdsChunk) {
        uint32_t ebyte[kW8A16LdsChunk][2];
        u32x4 xr[kW8A16LdsChunk][4];
#pragma unroll
        for (int c = 0; c < kW8A16LdsChunk; ++c) {
            const int64_t kb = kb0 + c * kStreamWaves;
            if (kb < kb_end) {
                ebyte[c][0] = erow[kb * 4];
                ebyte[c][1] = erow[kb * 4 + 2];
                if constexpr (kRegX) {
#pragma unroll
                    for (int j = 0; j < 4; ++j) xr[c][j] = load_16B(xreg + kb * 128 + (j < 2 ? 8 * j : 64 + 8 * (j - 2)));
                }
            }
        }
        if constexpr (!kRegX) {
#pragma unroll
            for (int c = 0; c < kW8A16LdsChunk; ++c) {
                const int64_t kb = kb0 + c * kStreamWaves;
                if (kb < kb_end) xrows_issue<kMp>(xrows[wave][c], rsrc_x, lane, K, kb);
            }
        }
#pragma unroll
        for (int c = 0; c < kW8A16LdsChunk; ++c) {
            const int64_t kb = kb0 + c * kStreamWaves;
            if (kb < kb_end) slab_issue(wslab[wave][c], rsrc_w, lane_off_w, K, kb, nt_loads);
        }
        const bool two = kb0 + kStreamWaves < kb_end;     // wave-uniform
#pragma unroll
        for (int c = 0; c < kW8A16LdsChunk; ++c) {
            const int64_t kb = kb0 + c * kStreamWaves;
            if (kb < kb_end) {
                wait_block(c, two);
                u32x4 wa0, wa1;
                slab_read(wslab[wave][c], r, g, wa0, wa1);
                const uint32_t q[8] = {wa0[0], wa0[1], wa0[2], wa0[3], wa1[0], wa1[1], wa1[2], wa1[3]};
                const uint8_t* row = xrows[wave][c] + r_row * kXRowStride + 32 * g;
                const float e0 = ue8m0_scale(ebyte[c][0]), e1 = ue8m0_scale(ebyte[c][1]);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    u32x4 xv;
                    if constexpr (kRegX) xv = xr[c][j];
                    else xv = *reinterpret_cast<const u32x4*>(row + (j < 2 ? 16 * j : 128 + 16 * (j - 2)));
                    xv = r_ok ? xv : z4;
                    const u32x4 a = widen8<false>(q[2 * j], q[2 * j + 1], j < 2 ? e0 : e1);
                    acc = mfma_f16_16x16x32(a, xv, acc);
                }
            }
        }
    }
    __syncthreads();   // every wave is done with the slabs that red overlays
    stream_finish(acc, red, y, y_dtype, M, N, nt, 0, splits, split, n_tiles, partials, counters);
}

// ------------------------------------------------- W8A16 all-token kernel ----
// The W8A16 product with every token of a group per workgroup (see
// w8a16_wide, w8a16_one_tile and blk32_wide for where it is used), for
// blk128 weights and for block-32 UE8M0 weights (kBlk32): a workgroup owns
// 16 kR weight rows (kR = 1 or 2, and 4 for blk128 with kT <= 2) and 16 kT
// tokens (kT = 1, 2 or 4 token tiles; grid.y walks further groups of 16 kT
// tokens) over all of K, so nothing is split across workgroups.
//
// A wave takes kTw of the kT token tiles (tiles kTw tg .. kTw tg + kTw - 1)
// and the 128-K blocks kw, kw + KW, ...: with G = kT / kTw token groups
// and kW waves, wave w has tg = w % G, kw = w / G, and KW = kW / G.  Where
// the LDS allows, every wave takes every token tile (kTw = kT, four waves;
// w16_wide_tiles_per_wave), so each block's weight rows are loaded and
// widened once per workgroup; one token tile and four tiles of two
// weight-row tiles run eight waves of one tile each, except that four
// weight-row tiles (8 KB of slabs a slot) always run four waves.
//
// Each wave owns a ring of LDS slots (two or three); a slot holds one
// block: the kR 16-row weight slabs (E4M3, 2 KB each), the wave's 16 kTw
// token rows (16-bit, 256 bytes each) and the block's weight scale word,
// all by direct-to-LDS loads of whole lines (16 bytes a lane; the scale
// word one dword).  Token row R of a tile keeps its 16-byte chunk c at
// position c ^ sw(R), sw(R) = ((R & 3) << 2) | (R >> 2), so the 16 rows of
// one MFMA read hit 16 distinct bank groups.  The weights are widened in
// registers (widen8) and feed four 16x16x32 MFMAs per block, row tile and
// token tile.  blk128: the block partial is promoted with the fp32 block
// scale, as in the streaming kernel.  Block-32: the scale word holds the
// four UE8M0 bytes of the block's 32x32 tiles in the row tile's 32-row band
// ([SM70] "How it works": one power-of-two scale per 32x32 tile), and each
// lane applies the two that cover its two 16-K chunks inside the widening,
// exactly, so the MFMAs accumulate across all of K with no promotion step,
// as in the block-32 streaming kernel.  The waves' partial sums meet in
// LDS once, at the end, and are added in K-lane order.
template <int kR, int kTw, int kW>
struct W16Slot {
    static constexpr int kOffX = kR * kSlabBytes;                  // 16 kTw token rows x 256 bytes
    static constexpr int kOffWs = kOffX + kTw * 16 * 256;
    static constexpr int kBytes = (kOffWs + 4 + 255) / 256 * 256;
    static constexpr int kSlotsFit = 160 * 1024 / (kW * kBytes);
    static constexpr int kSlots = kSlotsFit > 3 ? 3 : kSlotsFit;
    static constexpr int kVmem = 2 * kR + 4 * kTw + 1;             // load instructions per block
    static_assert(kSlots >= 2, "LDS ring");
};

template <int V, int Y>
__device__ __forceinline__ void w16_wait_n() {
    constexpr int n = Y * V;
    __builtin_amdgcn_s_waitcnt((n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

__device__ __forceinline__ int w16_sw(int row) { return ((row & 3) << 2) | ((row >> 2) & 3); }

template <bool kBlk32, bool kXBf16, int kT, int kR>
__global__ __launch_bounds__(w16_wide_waves(kR, kT) * kWave, 1) void w8a16_wide_kernel(
    const uint16_t* __restrict__ x, const uint8_t* __restrict__ wq, const void* __restrict__ scales,
    void* __restrict__ y, int y_dtype, int64_t M, int64_t N, int64_t K) {
    constexpr int kTw = w16_wide_tiles_per_wave(kR, kT), kW = w16_wide_waves(kR, kT);
    constexpr int G = kT / kTw, KW = kW / G;
    using SL = W16Slot<kR, kTw, kW>;
    constexpr int kW16WideSlots = SL::kSlots, kW16Slot = SL::kBytes, kW16OffX = SL::kOffX, kW16OffWs = SL::kOffWs;
    static_assert(kT == 1 || kT == 2 || kT == 4, "token tiles");
    static_assert(kT % kTw == 0 && kW % G == 0, "wave layout");
    static_assert(!kBlk32 || !kXBf16, "block-32 takes fp16 activations");
    static_assert(kR == 1 || kR == 2 || (kR == 4 && !kBlk32 && kT <= 2), "row tiles: one UE8M0 band, LDS slots");
    __shared__ __attribute__((aligned(1024))) uint8_t ring[kW * kW16WideSlots * kW16Slot];
    const int64_t nt = blockIdx.x, mg = blockIdx.y;
    const int KB = (int)(K / 128);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave), lane = threadIdx.x % kWave;
    const int tg = wave % G, kw = wave / G;
    const int r = lane & 15, g = lane >> 4;
    const int64_t m0 = 16 * kT * mg + 16 * kTw * tg;   // first token of this wave's tiles

    const int64_t n0 = 16 * kR * nt;
    const int64_t rows_w = N - n0 < 16 * kR ? N - n0 : 16 * kR;
    const i32x4 rsrc_w = buffer_rsrc(wq + n0 * K, (uint32_t)(rows_w * K));
    const int64_t rows_x = M - m0 > 0 ? (M - m0 < 16 * kTw ? M - m0 : 16 * kTw) : 0;
    const i32x4 rsrc_x = buffer_rsrc(x + m0 * K, (uint32_t)(rows_x * K * 2));
    // The block's scale word: the fp32 ws[n0 / 128, kb], or the UE8M0 bytes
    // of 32x32 tiles (n0 / 32, 4 kb .. 4 kb + 3) (K / 32 bytes a band, a
    // multiple of 4 since K % 128 == 0; the kR = 2 rows n0 = 32 nt .. +31
    // share one band).
    const i32x4 rsrc_ws =
        kBlk32 ? buffer_rsrc(static_cast<const uint8_t*>(scales) + (n0 / 32) * (K / 32), (uint32_t)(KB * 4))
               : buffer_rsrc(static_cast<const float*>(scales) + (n0 / 128) * KB, (uint32_t)(KB * 4));
    const int lane_off_w = slab_lane_offset(lane, K);
    // Token-row loads: instruction q covers rows 4q .. 4q + 3 (tile q / 4);
    // lane l fills position l % 16 of row 4q + l / 16 with logical chunk
    // (l % 16) ^ sw(row).
    int x_off[4 * kTw];
#pragma unroll
    for (int q = 0; q < 4 * kTw; ++q) {
        const int row = 4 * q + (lane >> 4);
        x_off[q] = (int)(row * K * 2) + (((lane & 15) ^ w16_sw(row)) << 4);
    }
    uint8_t* my_ring = ring + wave * kW16WideSlots * kW16Slot;

    auto issue = [&](int slot, int kb) {
        const uint32_t base = __builtin_amdgcn_readfirstlane(lds_address(my_ring + slot * kW16Slot));
        const int k_off = __builtin_amdgcn_readfirstlane(kb * 128);
        const int k_off_x = __builtin_amdgcn_readfirstlane(kb * 256);
#pragma unroll
        for (int q = 0; q < 2 * kR; ++q)
            dma16(base + 1024 * q, rsrc_w, lane_off_w, __builtin_amdgcn_readfirstlane((int)(8 * q * K)), k_off);
#pragma unroll
        for (int q = 0; q < 4 * kTw; ++q) dma16(base + kW16OffX + 1024 * q, rsrc_x, x_off[q], 0, k_off_x);
        if (lane == 0) dma4(base + kW16OffWs, rsrc_ws, 0, __builtin_amdgcn_readfirstlane(kb * 4));
    };

    const int nj = kw < KB ? (KB - 1 - kw) / KW + 1 : 0;
#pragma unroll
    for (int s = 0; s < kW16WideSlots; ++s)
        if (s < nj) issue(s, kw + KW * s);

    f32x4 acc[kR][kTw];
#pragma unroll
    for (int i = 0; i < kR; ++i)
#pragma unroll
        for (int t = 0; t < kTw; ++t) acc[i][t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    const f32x4 zero = {0.0f, 0.0f, 0.0f, 0.0f};
    const int sw = w16_sw(r);
    int slot = 0;
    for (int j = 0; j < nj; ++j) {
        const int younger = nj - 1 - j;
        if (kW16WideSlots > 2 && younger >= 2) w16_wait_n<SL::kVmem, (kW16WideSlots > 2 ? 2 : 1)>();
        else if (younger >= 1) w16_wait_n<SL::kVmem, 1>();
        else w16_wait_n<SL::kVmem, 0>();
        asm volatile("" ::: "memory");
        const uint8_t* sl = my_ring + slot * kW16Slot;
        u32x4 wa0[kR], wa1[kR];
#pragma unroll
        for (int i = 0; i < kR; ++i) slab_read(sl + i * kSlabBytes, r, g, wa0[i], wa1[i]);
        // MFMA i takes K offsets 16 g + 8 i (i < 2) and 64 + 16 g + 8 (i - 2):
        // 16-bit chunks 2 g + i and 8 + 2 g + (i - 2) of the token row.
        u32x4 xv[kTw][4];
#pragma unroll
        for (int t = 0; t < kTw; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int c = i < 2 ? 2 * g + i : 8 + 2 * g + (i - 2);
                xv[t][i] = *reinterpret_cast<const u32x4*>(sl + kW16OffX + t * 4096 + r * 256 + ((c ^ sw) << 4));
            }
        const uint32_t sword = *reinterpret_cast<const uint32_t*>(sl + kW16OffWs);
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        if (j + kW16WideSlots < nj) issue(slot, kw + KW * (j + kW16WideSlots));
#pragma unroll
        for (int rt = 0; rt < kR; ++rt) {
            const uint32_t q8[8] = {wa0[rt][0], wa0[rt][1], wa0[rt][2], wa0[rt][3],
                                    wa1[rt][0], wa1[rt][1], wa1[rt][2], wa1[rt][3]};
            if constexpr (kBlk32) {
                // Chunk g (K 16 g .. 16 g + 15) lies in tile 4 kb + g / 2,
                // chunk g + 4 in tile 4 kb + 2 + g / 2.
                const float e0 = ue8m0_scale((sword >> (8 * (g >> 1))) & 0xFF);
                const float e1 = ue8m0_scale((sword >> (8 * (2 + (g >> 1)))) & 0xFF);
                u32x4 a[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) a[i] = widen8<false>(q8[2 * i], q8[2 * i + 1], i < 2 ? e0 : e1);
#pragma unroll
                for (int t = 0; t < kTw; ++t)
#pragma unroll
                    for (int i = 0; i < 4; ++i) acc[rt][t] = mfma_f16_16x16x32(a[i], xv[t][i], acc[rt][t]);
            } else {
                u32x4 a[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) a[i] = widen8<kXBf16>(q8[2 * i], q8[2 * i + 1]);
                const float sc = __builtin_bit_cast(float, sword);
#pragma unroll
                for (int t = 0; t < kTw; ++t) {
                    f32x4 blk = zero;
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        blk = kXBf16 ? mfma_bf16_16x16x32(a[i], xv[t][i], blk) : mfma_f16_16x16x32(a[i], xv[t][i], blk);
#pragma unroll
                    for (int e = 0; e < 4; ++e) acc[rt][t][e] = __builtin_fmaf(blk[e], sc, acc[rt][t][e]);
                }
            }
        }
        slot = slot + 1 == kW16WideSlots ? 0 : slot + 1;
    }

    __syncthreads();
    float* red = reinterpret_cast<float*>(ring);
#pragma unroll
    for (int i = 0; i < kR; ++i)
#pragma unroll
        for (int t = 0; t < kTw; ++t)
            *reinterpret_cast<f32x4*>(red + (((kw * kR + i) * kT + kTw * tg + t) * kWave + lane) * 4) = acc[i][t];
    __syncthreads();
    const int L = threadIdx.x % kWave, rr = L & 15, gg = L >> 4;
    for (int u = threadIdx.x / kWave; u < kR * kT; u += kW) {
        f32x4 v = *reinterpret_cast<const f32x4*>(red + (u * kWave + L) * 4);
#pragma unroll
        for (int w = 1; w < KW; ++w) v += *reinterpret_cast<const f32x4*>(red + ((w * kR * kT + u) * kWave + L) * 4);
        const int i = u / kT, tt = u % kT;
        const int64_t m = 16 * kT * mg + 16 * tt + rr;
        const int64_t n = n0 + 16 * i + 4 * gg;
        if (m < M && n < N) {
            const int64_t idx = m * N + n;
            if (y_dtype == 2) {
                *reinterpret_cast<f32x4*>(static_cast<float*>(y) + idx) = v;
            } else {
                uint32_t h[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) h[e] = y_dtype == 0 ? float_to_bf16_bits(v[e]) : float_to_f16_bits(v[e]);
                *reinterpret_cast<uint2*>(static_cast<uint16_t*>(y) + idx) = make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
            }
        }
    }
}

#define BFP8_LAUNCH_W16(S, B, T, R)                                                                       \
    hipLaunchKernelGGL((w8a16_wide_kernel<S, B, T, R>), grid, dim3(w16_wide_waves(R, T) * kWave), 0, stream, xh, \
                       wq, scales, y, y_dtype, M, N, K)
// kr = 4 (blk128, kt <= 2 only) is instantiated only where it can run.
#define BFP8_LAUNCH_W16_KR(S, B, T)                                                     \
    if (w.kr == 1) BFP8_LAUNCH_W16(S, B, T, 1);                                         \
    else if (w.kr == 2 || (S) || (T) == 4) BFP8_LAUNCH_W16(S, B, T, 2);                 \
    else BFP8_LAUNCH_W16(S, B, T, ((S) || (T) == 4 ? 2 : 4));

hipError_t launch_w8a16_wide(const void* x, bool x_bf16, const uint8_t* wq, const float* ws, void* y, int y_dtype,
                             int64_t M, int64_t N, int64_t K, hipStream_t stream) {
    if (M < 1 || N % 16 != 0 || K > kTileMaxK) return hipErrorInvalidValue;
    const WideShape w = w16_wide_shape(M, N);
    if (w.groups_m > 65535 || (w.kr == 4 && w.kt > 2)) return hipErrorInvalidValue;
    const dim3 grid(w.groups_n, w.groups_m);
    const uint16_t* xh = static_cast<const uint16_t*>(x);
    const void* scales = ws;
    if (x_bf16) {
        if (w.kt == 1) { BFP8_LAUNCH_W16_KR(false, true, 1) }
        else if (w.kt == 2) { BFP8_LAUNCH_W16_KR(false, true, 2) }
        else { BFP8_LAUNCH_W16_KR(false, true, 4) }
    } else {
        if (w.kt == 1) { BFP8_LAUNCH_W16_KR(false, false, 1) }
        else if (w.kt == 2) { BFP8_LAUNCH_W16_KR(false, false, 2) }
        else { BFP8_LAUNCH_W16_KR(false, false, 4) }
    }
    return hipGetLastError();
}

hipError_t launch_w8a16_blk32_wide(const void* x, const uint8_t* wq, const uint8_t* e8m0, void* y, int y_dtype,
                                   int64_t M, int64_t N, int64_t K, hipStream_t stream) {
    if (M < 1 || N % 32 != 0 || K % 128 != 0 || K > kTileMaxK) return hipErrorInvalidValue;
    const WideShape w = blk32_wide_shape(M, N);
    if (w.groups_m > 65535 || w.kr > 2) return hipErrorInvalidValue;
    const dim3 grid(w.groups_n, w.groups_m);
    const uint16_t* xh = static_cast<const uint16_t*>(x);
    const void* scales = e8m0;
    if (w.kt == 1) { BFP8_LAUNCH_W16_KR(true, false, 1) }
    else if (w.kt == 2) { BFP8_LAUNCH_W16_KR(true, false, 2) }
    else { BFP8_LAUNCH_W16_KR(true, false, 4) }
    return hipGetLastError();
}
#undef BFP8_LAUNCH_W16_KR
#undef BFP8_LAUNCH_W16

// ------------------------------------------------ W8A16 GEMV, M = 1 ----
// One token (batch-1 decode) needs no matrix core: the work is one dot
// product per weight row.  A wave owns one weight row.  Lane l takes, in
// each 1 KB chunk c of the row, the 16 weight bytes at K offset
// 1024 c + 16 l (one load instruction covers 8 whole 128-byte lines) and the
// 16 matching activations, widens the E4M3 weights to the activations'
// 16-bit type (exact) and sums the 16 products with v_dot2c (lane_dot16).
// Lanes 8 j .. 8 j + 7 hold 128-K block 8 c + j: three lane exchanges give
// every one of them the block's dot product, which is promoted once with
// the block's weight scale (the per-block promotion of [ARC] "What this
// adds", here without a matrix instruction).  The eight lane groups'
// promoted sums are added at the end (three more exchanges, inside the ALU)
// and lane 0 stores the row.  Every load is issued before the first product
// and the token is shared through LDS (stream_common.hpp); there is no
// cross-wave reduction, which costs the streaming kernel about half a
// microsecond of a 5.7 us launch at N = K = 4096 (the first, four-wave form
// of this kernel measured 5.33-5.42 vs 5.69 us there, 3.00 vs 3.96 us at
// N = 1024 and 11.1 vs 11.5 us at N = 12288).  Lanes past K read zeros
// (their offsets are moved past the descriptor's range).

// A lane's 16 activations of a chunk (two 16-byte loads) as 8 pairs.
__device__ __forceinline__ const uint32_t (&pairs(const i32x4 (&x)[2]))[8] {
    return *reinterpret_cast<const uint32_t(*)[8]>(&x[0]);
}

template <bool kXBf16, int kC, int kPol>
__global__ __launch_bounds__(kGemvThreads) void w8a16_gemv_kernel(
    const uint16_t* __restrict__ x, const uint8_t* __restrict__ wq, const float* __restrict__ ws,
    void* __restrict__ y, int y_dtype, int64_t N, int64_t K) {
    constexpr int kU = kC / 4;   // 8 KB rounds of the 16-bit token (2 KB per chunk)
    __shared__ __attribute__((aligned(16))) uint8_t x_lds[2048 * kC];
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave), lane = threadIdx.x % kWave;
    const int64_t n = (int64_t)blockIdx.x * kGemvWaves + wave;   // wave-uniform: scalar descriptors
    // The launch covers N exactly (N % 16 == 0); a wave past N would still
    // take part in the token copy and the barrier, with empty descriptors.
    const bool live = n < N;
    const int64_t nb = live ? n : 0;
    const int KB = (int)(K / 128);
    const __amdgpu_buffer_rsrc_t rw =
        __builtin_amdgcn_make_buffer_rsrc((void*)(wq + nb * K), 0, live ? (int)K : 0, 0x00020000);
    const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc((void*)x, 0, (int)(2 * K), 0x00020000);
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc((void*)(ws + (nb / 128) * KB), 0, live ? KB * 4 : 0, 0x00020000);

    i32x4 xr[kU], wv[kC];
    float wsv[kC];
    gemv_x_issue<kU>(rx, xr);
#pragma unroll
    for (int c = 0; c < kC; ++c)
        wsv[c] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, 4 * ((1024 * c + 16 * lane) / 128), 0, 0));
#pragma unroll
    for (int c = 0; c < kC; ++c) {
        const int k = 1024 * c + 16 * lane;
        wv[c] = __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(rw, k < K ? k : (int)K, 0, kPol));
    }
    // Keep every load ahead of the token copy and the arithmetic: the
    // scheduler would otherwise sink the later chunks' loads below the
    // first chunk's products.
    __builtin_amdgcn_sched_barrier(0);
    gemv_x_store<kU>(x_lds, xr);
    __syncthreads();

    float acc = 0.0f;
#pragma unroll
    for (int c = 0; c < kC; ++c) {
        // Lane l's 16 activations of chunk c: bytes 2048 c + 32 l .. + 31.
        // Chunks past K hold zeros only (weights and token), so they add
        // nothing and need no branch.
        const i32x4 xv[2] = {gemv_x_read(x_lds, 128 * c + 2 * lane), gemv_x_read(x_lds, 128 * c + 2 * lane + 1)};
        acc = __builtin_fmaf(block_sum8(lane_dot16<kXBf16>(pairs(xv), wv[c])), wsv[c], acc);
    }
    const float v = group_sum8(acc);
    if (lane == 0 && live) store_out(y, y_dtype, n, v);
}

// Block-32 UE8M0 weights, one token ([SM70] "How it works": a GEMV for the
// fewest tokens): the one-token layout above with fp16 activations.  A
// lane's 16 weights of a chunk lie in one 32-wide K tile (16 divides 32), so
// they share one scale 2^e, which the conversion applies: each weight
// becomes the fp16 number value * 2^e exactly, the lane's 16 products (each
// exact in fp32) are summed by v_dot2c, and the lane totals over the wave in
// one fixed order.  The scale byte E (e = E - 127) of lane l in chunk c is
// e8m0[n / 32, 32 c + l / 2].
template <int kC, int kPol>
__global__ __launch_bounds__(kGemvThreads) void w8a16_blk32_gemv_kernel(
    const uint16_t* __restrict__ x, const uint8_t* __restrict__ wq, const uint8_t* __restrict__ e8m0,
    void* __restrict__ y, int y_dtype, int64_t N, int64_t K) {
    constexpr int kU = kC / 4;
    __shared__ __attribute__((aligned(16))) uint8_t x_lds[2048 * kC];
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave), lane = threadIdx.x % kWave;
    const int64_t n = (int64_t)blockIdx.x * kGemvWaves + wave;   // wave-uniform: scalar descriptors
    const bool live = n < N;                                      // as in w8a16_gemv_kernel
    const int64_t nb = live ? n : 0;
    const int K32 = (int)(K / 32);
    const __amdgpu_buffer_rsrc_t rw =
        __builtin_amdgcn_make_buffer_rsrc((void*)(wq + nb * K), 0, live ? (int)K : 0, 0x00020000);
    const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc((void*)x, 0, (int)(2 * K), 0x00020000);
    const __amdgpu_buffer_rsrc_t re =
        __builtin_amdgcn_make_buffer_rsrc((void*)(e8m0 + (nb / 32) * K32), 0, live ? K32 : 0, 0x00020000);

    i32x4 xr[kU], wv[kC];
    uint32_t eb[kC];
    gemv_x_issue<kU>(rx, xr);
#pragma unroll
    for (int c = 0; c < kC; ++c) eb[c] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(re, (1024 * c + 16 * lane) / 32, 0, 0);
#pragma unroll
    for (int c = 0; c < kC; ++c) {
        const int k = 1024 * c + 16 * lane;
        wv[c] = __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(rw, k < K ? k : (int)K, 0, kPol));
    }
    __builtin_amdgcn_sched_barrier(0);   // every load ahead of the token copy and the arithmetic
    gemv_x_store<kU>(x_lds, xr);
    __syncthreads();

    float acc = 0.0f;
#pragma unroll
    for (int c = 0; c < kC; ++c) {
        const i32x4 xv[2] = {gemv_x_read(x_lds, 128 * c + 2 * lane), gemv_x_read(x_lds, 128 * c + 2 * lane + 1)};
        // 2^(E - 127) (E in [113, 134]) goes into the widening: each weight
        // becomes the fp16 number value * 2^e exactly.  Lanes past K read
        // E = 0 and zero weights, which widen to zeros.
        acc += lane_dot16<false>(pairs(xv), wv[c], ue8m0_scale(eb[c]));
    }
    const float v = wave_sum(acc);
    if (lane == 0 && live) store_out(y, y_dtype, n, v);
}

hipError_t launch_w8a16_gemv(const void* x, bool x_bf16, const uint8_t* wq, const float* ws, void* y, int y_dtype,
                             int64_t N, int64_t K, hipStream_t stream) {
    if (N % 16 != 0 || K > kGemvMaxK) return hipErrorInvalidValue;
    const dim3 grid((unsigned)((N + kGemvWaves - 1) / kGemvWaves));
    const uint16_t* xh = static_cast<const uint16_t*>(x);
#define BFP8_LAUNCH_GEMV(B, C, P)                                                                                  \
    hipLaunchKernelGGL((w8a16_gemv_kernel<B, C, P>), grid, dim3(kGemvThreads), 0, stream, xh, wq, ws, y, y_dtype, N, K)
#define BFP8_LAUNCH_GEMV_C(B, P)                    \
    switch (gemv_chunks(K)) {                        \
        case 4: BFP8_LAUNCH_GEMV(B, 4, P); break;   \
        case 8: BFP8_LAUNCH_GEMV(B, 8, P); break;   \
        case 12: BFP8_LAUNCH_GEMV(B, 12, P); break; \
        default: BFP8_LAUNCH_GEMV(B, 16, P); break; \
    }
    const bool nt = weights_nt(N, K);
    if (x_bf16) {
        if (nt) { BFP8_LAUNCH_GEMV_C(true, kLoadNt) }
        else { BFP8_LAUNCH_GEMV_C(true, 0) }
    } else {
        if (nt) { BFP8_LAUNCH_GEMV_C(false, kLoadNt) }
        else { BFP8_LAUNCH_GEMV_C(false, 0) }
    }
#undef BFP8_LAUNCH_GEMV_C
#undef BFP8_LAUNCH_GEMV
    return hipGetLastError();
}

hipError_t launch_w8a16_blk32_gemv(const void* x, const uint8_t* wq, const uint8_t* e8m0, void* y, int y_dtype,
                                   int64_t N, int64_t K, hipStream_t stream) {
    if (N % 32 != 0 || K > kGemvMaxK) return hipErrorInvalidValue;
    const dim3 grid((unsigned)((N + kGemvWaves - 1) / kGemvWaves));
    const uint16_t* xh = static_cast<const uint16_t*>(x);
#define BFP8_LAUNCH_GEMV32(C, P)                                                                                  \
    hipLaunchKernelGGL((w8a16_blk32_gemv_kernel<C, P>), grid, dim3(kGemvThreads), 0, stream, xh, wq, e8m0, y,        \
                       y_dtype, N, K)
#define BFP8_LAUNCH_GEMV32_C(P)                    \
    switch (gemv_chunks(K)) {                       \
        case 4: BFP8_LAUNCH_GEMV32(4, P); break;   \
        case 8: BFP8_LAUNCH_GEMV32(8, P); break;   \
        case 12: BFP8_LAUNCH_GEMV32(12, P); break; \
        default: BFP8_LAUNCH_GEMV32(16, P); break; \
    }
    if (weights_nt(N, K)) { BFP8_LAUNCH_GEMV32_C(kLoadNt) }
    else { BFP8_LAUNCH_GEMV32_C(0) }
#undef BFP8_LAUNCH_GEMV32_C
#undef BFP8_LAUNCH_GEMV32
    return hipGetLastError();
}

hipError_t launch_w8a16_blk128_stream(const void* x, bool x_bf16, const uint8_t* wq, const float* ws,
                                      void* y, int y_dtype, int64_t M, int64_t N, int64_t K,
                                      void* workspace, hipStream_t stream) {
    const StreamPlan p = plan_stream(M, N, K);
    uint32_t* counters;
    float* partials;
    if (!stream_workspace_parts(p, workspace, counters, partials)) return hipErrorInvalidValue;
    const dim3 grid((unsigned)p.n_tiles, (unsigned)p.splits, (unsigned)p.m_tiles);
    if (M <= kW8A16LdsMaxM) {
        const int mp = M <= 1 ? 1 : M <= 2 ? 2 : M <= 4 ? 4 : M <= 8 ? 8 : 16;
        const uint16_t* xh = static_cast<const uint16_t*>(x);
#define BFP8_LAUNCH_LDS(BF, MP)                                                                                \
    hipLaunchKernelGGL((w8a16_blk128_stream_lds_kernel<BF, MP>), grid, dim3(kStreamThreads), 0, stream, xh, wq, ws, \
                       y, y_dtype, M, N, K, p.n_tiles, p.splits, p.kb_per_split, partials, counters)
        if (x_bf16) {
            switch (mp) {
                case 1: BFP8_LAUNCH_LDS(true, 1); break;
                case 2: BFP8_LAUNCH_LDS(true, 2); break;
                case 4: BFP8_LAUNCH_LDS(true, 4); break;
                case 8: BFP8_LAUNCH_LDS(true, 8); break;
                default: BFP8_LAUNCH_LDS(true, 16); break;
            }
        } else {
            switch (mp) {
                case 1: BFP8_LAUNCH_LDS(false, 1); break;
                case 2: BFP8_LAUNCH_LDS(false, 2); break;
                case 4: BFP8_LAUNCH_LDS(false, 4); break;
                case 8: BFP8_LAUNCH_LDS(false, 8); break;
                default: BFP8_LAUNCH_LDS(false, 16); break;
            }
        }
#undef BFP8_LAUNCH_LDS
        return hipGetLastError();
    }
    return hipErrorInvalidValue;   // M > 16 runs the tiled kernel (launch_w8a16_tile)
}

hipError_t launch_w8a16_blk32_stream(const void* x, const uint8_t* wq, const uint8_t* e8m0,
                                     void* y, int y_dtype, int64_t M, int64_t N, int64_t K,
                                     void* workspace, hipStream_t stream) {
    const StreamPlan p = plan_stream(M, N, K);
    uint32_t* counters;
    float* partials;
    if (!stream_workspace_parts(p, workspace, counters, partials)) return hipErrorInvalidValue;
    if (M <= kW8A16LdsMaxM) {
        const dim3 grid((unsigned)p.n_tiles, (unsigned)p.splits, 1u);
        const uint16_t* xh = static_cast<const uint16_t*>(x);
#define BFP8_LAUNCH_LDS32(MP)                                                                                   \
    hipLaunchKernelGGL(w8a16_blk32_stream_lds_kernel<MP>, grid, dim3(kStreamThreads), 0, stream, xh, wq, e8m0, y, \
                       y_dtype, M, N, K, p.n_tiles, p.splits, p.kb_per_split, partials, counters)
        switch (M <= 1 ? 1 : M <= 2 ? 2 : M <= 4 ? 4 : M <= 8 ? 8 : 16) {
            case 1: BFP8_LAUNCH_LDS32(1); break;
            case 2: BFP8_LAUNCH_LDS32(2); break;
            case 4: BFP8_LAUNCH_LDS32(4); break;
            case 8: BFP8_LAUNCH_LDS32(8); break;
            default: BFP8_LAUNCH_LDS32(16); break;
        }
#undef BFP8_LAUNCH_LDS32
        return hipGetLastError();
    }
    hipLaunchKernelGGL(w8a16_blk32_stream_kernel, dim3((unsigned)p.n_tiles, (unsigned)p.splits, (unsigned)p.m_tiles),
                       dim3(kStreamThreads), 0, stream, static_cast<const uint16_t*>(x), wq, e8m0, y, y_dtype,
                       M, N, K, p.n_tiles, p.splits, p.kb_per_split, partials, counters);
    return hipGetLastError();
}

}  // namespace bfp8
