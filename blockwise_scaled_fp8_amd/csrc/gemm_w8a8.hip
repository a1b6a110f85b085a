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
// Three kernels, chosen by M ([ADA] "One tile doesn't fit all M"):
//   * stream (M <= 16, or up to 64 on small projections; see w8a8_streams):
//     weight streaming.  One workgroup per 16 weight rows and 16-token tile
//     (and per split of K), sixteen waves each holding its 128-K blocks of
//     weight loads in flight, tokens padded to 16 on the MFMA column axis.
//   * wide (M <= 64, see w8a8_wide): one workgroup per 16 weight rows and
//     all tokens over all of K, eight waves with private LDS rings.
//   * tile (larger M): in gemm_w8a8_tile.hip.

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
    // K is split over workgroups only when it is long (more than 64 blocks,
    // more than two passes of two blocks per wave): up to K = 8192 a single
    // pass with every load in flight at once beats the split-K hand-off even
    // with few workgroups (measured, us, K split vs not: N = 1024, K = 4096,
    // M = 1 / 8 / 16: 5.4 / 5.6 / 5.8 vs 3.3 / 4.0 / 4.5; N = 512, M = 1:
    // 4.7 vs 3.3; N = 1024, K = 8192: 6.2 vs 4.4), while at K = 12288 the
    // serial passes cost more (N = 1024, M = 16: 7.5 vs 11.5).  Then: enough
    // workgroups to give each of the 256 CUs one, while at least half of a
    // workgroup's waves still get a 128-K block.
    const int64_t tiles = p.n_tiles * p.m_tiles;
    int64_t splits = 1;
    while (KB > 64 && tiles * splits < 256 && 2 * (KB / (splits * 2)) >= kStreamWaves) splits *= 2;
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

// Lane (r, g) supplies weight row n0 + r and token m0 + r; of each 128-K
// block it holds the 16-byte chunks g and g + 4 (K offsets 16g and 64 + 16g),
// the same for both MFMA operands.  The waves take interleaved 128-K blocks,
// so at any time a workgroup reads adjacent blocks of its rows.
//
// M <= 16 (padded token count Mp = 1, 2, 4, 8 or 16): the same product
// with both operands staged in LDS.  The weights arrive as whole 128-byte
// lines in per-wave slabs; the block's token rows (128 code bytes each) by
// direct-to-LDS dword loads, two rows per load, lane l of a load fetching
// the dword that belongs at LDS position 4 l of the two 128-byte rows with
// the slab's chunk swizzle (chunk c of row R at position c ^ (R & 7)), so the
// MFMA operand reads back with slab_read.  Rows past M lie outside the
// buffer descriptor and read as zeros.  Per wave and block that is two
// weight loads and Mp / 2 token loads (one for Mp = 1), against two
// half-line weight loads and two 16-byte token loads per lane in the kernel
// above; the token scales stay register loads (one dword per lane).
template <int kMp>
__device__ __forceinline__ void code_rows_issue(uint8_t* rows, i32x4 rsrc_x, int lane, int64_t K, int64_t kb) {
    const uint32_t base = __builtin_amdgcn_readfirstlane(lds_address(rows));
    const int k_off = __builtin_amdgcn_readfirstlane((int)(kb * 128));
    const int p = (lane & 31) >> 2;   // 16-byte chunk position inside the row
#pragma unroll
    for (int i = 0; i < (kMp + 1) / 2; ++i) {
        const int row = 2 * i + (lane >> 5);
        const int voff = (int)(row * K) + 16 * (p ^ (row & 7)) + 4 * (lane & 3);
        dma4(__builtin_amdgcn_readfirstlane(base + 256 * i), rsrc_x, voff, k_off);
    }
}

constexpr int kCodesLdsChunk = 2;
static_assert(kCodesLdsChunk == 2, "wait_block counts two blocks per pass");

template <int kMp>
__global__ __launch_bounds__(kStreamThreads) void w8a8_stream_lds_kernel(
    const uint8_t* __restrict__ xq, const float* __restrict__ xs,
    const uint8_t* __restrict__ wq, const float* __restrict__ ws,
    void* __restrict__ y, int y_dtype, int64_t M, int64_t N, int64_t K,
    int64_t n_tiles, int64_t splits, int64_t kb_per_split,
    float* __restrict__ partials, uint32_t* __restrict__ counters) {
    constexpr int kRowsBytes = (kMp + 1) / 2 * 256;
    __shared__ __attribute__((aligned(1024))) uint8_t xrows[kStreamWaves][kCodesLdsChunk][kRowsBytes];
    __shared__ __attribute__((aligned(1024))) uint8_t wslab[kStreamWaves][kCodesLdsChunk][kSlabBytes];
    float* red = slab_scratch(&wslab[0][0][0]);   // used after the last block only
    // Token tile mt = blockIdx.z: tokens m0 .. m0 + Mt - 1.  With one token
    // tile no other workgroup reads these weights: non-temporal loads when
    // they are large enough (weights_nt).
    const int64_t nt = blockIdx.x, split = blockIdx.y, mt = blockIdx.z;
    const int64_t m0 = 16 * mt, Mt = M - m0 < 16 ? M - m0 : 16;
    const bool nt_loads = gridDim.z == 1 && weights_nt(N, K);
    const int64_t KB = K / 128;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave), lane = threadIdx.x % kWave;
    const int r = lane & 15, g = lane >> 4;
    const bool r_ok = r < kMp && r < Mt;
    const int r_row = r < kMp ? r : 0;
    const int64_t kb_begin = split * kb_per_split;
    const int64_t kb_end = kb_begin + kb_per_split < KB ? kb_begin + kb_per_split : KB;

    const i32x4 rsrc_w = buffer_rsrc(wq + nt * 16 * K, (uint32_t)(16 * K));
    const i32x4 rsrc_x = buffer_rsrc(xq + m0 * K, (uint32_t)(Mt * K));
    const int lane_off_w = slab_lane_offset(lane, K);
    const float* ws_row = ws + (nt * 16 / 128) * KB;
    const float* xs_row = xs + (m0 + (r_ok ? r : 0)) * KB;   // rows past M read row m0, zeroed at use

    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
    const f32x4 zero = {0.0f, 0.0f, 0.0f, 0.0f};
    const u32x4 z4 = {0u, 0u, 0u, 0u};
    for (int64_t kb0 = kb_begin + wave; kb0 < kb_end; kb0 += kStreamWaves * kCodesLdsChunk) {
        float xsv[kCodesLdsChunk], wsv[kCodesLdsChunk];
#pragma unroll
        for (int c = 0; c < kCodesLdsChunk; ++c) {
            const int64_t kb = kb0 + c * kStreamWaves;
            if (kb < kb_end) {
                xsv[c] = xs_row[kb];
                wsv[c] = ws_row[kb];
            }
        }
#pragma unroll
        for (int c = 0; c < kCodesLdsChunk; ++c) {
            const int64_t kb = kb0 + c * kStreamWaves;
            if (kb < kb_end) code_rows_issue<kMp>(xrows[wave][c], rsrc_x, lane, K, kb);
        }
#pragma unroll
        for (int c = 0; c < kCodesLdsChunk; ++c) {
            const int64_t kb = kb0 + c * kStreamWaves;
            if (kb < kb_end) slab_issue(wslab[wave][c], rsrc_w, lane_off_w, K, kb, nt_loads);
        }
        const bool two = kb0 + kStreamWaves < kb_end;     // wave-uniform
#pragma unroll
        for (int c = 0; c < kCodesLdsChunk; ++c) {
            const int64_t kb = kb0 + c * kStreamWaves;
            if (kb < kb_end) {
                wait_block(c, two);
                u32x4 wa0, wa1, b0, b1;
                slab_read(wslab[wave][c], r, g, wa0, wa1);
                slab_read(xrows[wave][c], r_row, g, b0, b1);
                b0 = r_ok ? b0 : z4;
                b1 = r_ok ? b1 : z4;
                const i32x8 a = __builtin_bit_cast(i32x8, __builtin_shufflevector(wa0, wa1, 0, 1, 2, 3, 4, 5, 6, 7));
                const i32x8 b = __builtin_bit_cast(i32x8, __builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7));
                const f32x4 blk = mfma_e4m3_16x16x128(a, b, zero);
                const float sc = r_ok ? xsv[c] * wsv[c] : 0.0f;
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[i] = __builtin_fmaf(blk[i], sc, acc[i]);
            }
        }
    }
    __syncthreads();   // every wave is done with the slabs that red overlays
    stream_finish(acc, red, y, y_dtype, M, N, nt, mt, splits, split, n_tiles, partials, counters);
}

// ------------------------------------------- activation quant fused in ----
// The same streaming GEMM for M <= kFusedQuantMaxM with 16-bit activations
// in: each wave quantises, for every 128-K block it multiplies, the block's
// 1x128 groups of the (at most 8) tokens itself.  [ADA] "Results on the L4"
// counts the activation quantisation inside the kernel's time, and "What's
// not good yet" names batch-1 decode, memory-bound, as the remaining gap;
// fusing removes a launch and the codes' round trip through memory there.
//
// Load order per wave: the weight scales, then the block's token rows
// (direct-to-LDS dword loads, 256 bytes per token row; rows past M lie
// outside the buffer descriptor and read as zeros), then the weight slabs.
// Loads complete in issue order, so the wave waits for its token rows with
// the weight loads still in flight and quantises while the weights stream
// from HBM; only the MFMA and the promotion are left for after the weights
// arrive.  The 64 lanes split the padded token count Mp (1, 2, 4 or 8)
// evenly: 64/Mp lanes per token, 2 Mp values per lane, so no lane quantises
// padding when M is small.  The group maximum is a butterfly over the
// token's lanes; scale, quotients and codes use the quantiser's own
// arithmetic (quantize_v), so codes, scales and results are bit-identical to
// bfp8_quantize_act_1x128 followed by the codes kernel.  The codes overwrite
// the first 128 bytes of their token row in LDS (a wave's LDS accesses run in
// issue order, and every lane has read its values before any lane writes),
// and are read back in the MFMA operand layout.
constexpr int kFusedChunk = 2;
template <int NW>
__device__ __forceinline__ void read_words(const uint8_t* p, uint32_t (&w)[NW]) {
    if constexpr (NW == 1) {
        w[0] = *reinterpret_cast<const uint32_t*>(p);
    } else if constexpr (NW == 2) {
        const uint2 v = *reinterpret_cast<const uint2*>(p);
        w[0] = v.x;
        w[1] = v.y;
    } else {
#pragma unroll
        for (int i = 0; i < NW / 4; ++i) {
            const u32x4 v = *reinterpret_cast<const u32x4*>(p + 16 * i);
#pragma unroll
            for (int e = 0; e < 4; ++e) w[4 * i + e] = v[e];
        }
    }
}

template <int NB>
__device__ __forceinline__ void store_codes(uint8_t* p, const uint32_t (&c)[(NB + 3) / 4]) {
    if constexpr (NB == 2) {
        *reinterpret_cast<uint16_t*>(p) = (uint16_t)c[0];
    } else if constexpr (NB == 4) {
        *reinterpret_cast<uint32_t*>(p) = c[0];
    } else if constexpr (NB == 8) {
        *reinterpret_cast<uint2*>(p) = make_uint2(c[0], c[1]);
    } else {
        *reinterpret_cast<u32x4*>(p) = u32x4{c[0], c[1], c[2], c[3]};
    }
}

// Maximum over each token's kL lanes (aligned groups of 8, 16, 32 or 64):
// DPP within rows of 16 lanes, then the row maxima read as scalars.
template <int kL>
__device__ __forceinline__ float token_max(float v) {
    if constexpr (kL <= 16) {
        return group_max_dpp<kL>(v);
    } else {
        v = group_max_dpp<16>(v);
        const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
        const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
        const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
        const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
        if constexpr (kL == 64) return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
        else return (threadIdx.x & 32) ? fmaxf(r2, r3) : fmaxf(r0, r1);
    }
}

// Value v of token t's first lane (lane t * 64 / kMp), for token t = `tok`.
template <int kMp>
__device__ __forceinline__ float token_value(float v, int tok) {
    constexpr int kL = kWave / kMp;
    float out = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
#pragma unroll
    for (int t = 1; t < kMp; ++t) {
        const float vt = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), t * kL));
        out = tok == t ? vt : out;
    }
    return out;
}

template <bool kBf16, int kMp>
__global__ __launch_bounds__(kStreamThreads) void w8a8_stream_quant_kernel(
    const uint16_t* __restrict__ x, const uint8_t* __restrict__ wq, const float* __restrict__ ws,
    void* __restrict__ y, int y_dtype, int64_t M, int64_t N, int64_t K,
    int64_t n_tiles, int64_t splits, int64_t kb_per_split,
    float* __restrict__ partials, uint32_t* __restrict__ counters) {
    constexpr int kL = kWave / kMp;          // lanes per token
    constexpr int kV = 128 / kL;             // values per lane (2 Mp)
    static_assert(kFusedChunk == 2, "the token-row wait counts two slab loads per block");
    __shared__ __attribute__((aligned(16))) uint8_t xrows[kStreamWaves][kFusedChunk][kMp * kXRowStride];
    __shared__ __attribute__((aligned(1024))) uint8_t wslab[kStreamWaves][kFusedChunk][kSlabBytes];
    float* red = slab_scratch(&wslab[0][0][0]);   // used after the last block only
    const int64_t nt = blockIdx.x, split = blockIdx.y;
    const bool nt_loads = weights_nt(N, K);   // M <= 8: one token tile, no other workgroup reads these weights
    const int64_t KB = K / 128;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave), lane = threadIdx.x % kWave;
    const int r = lane & 15, g = lane >> 4;
    const int64_t kb_begin = split * kb_per_split;
    const int64_t kb_end = kb_begin + kb_per_split < KB ? kb_begin + kb_per_split : KB;

    // Quantiser role: token qt, values [qp * kV, qp * kV + kV) of each block.
    const int qt = lane / kL, qp = lane % kL;
    // MFMA role: weight row n0 + r, token r (rows r >= kMp are padding).
    const bool r_ok = r < kMp;
    const int r_row = r_ok ? r : 0;
    const i32x4 rsrc_w = buffer_rsrc(wq + nt * 16 * K, (uint32_t)(16 * K));
    const i32x4 rsrc_x = buffer_rsrc(x, (uint32_t)(M * K * 2));
    const int lane_off_w = slab_lane_offset(lane, K);
    const float* ws_row = ws + (nt * 16 / 128) * KB;

    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
    const f32x4 zero = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int64_t kb0 = kb_begin + wave; kb0 < kb_end; kb0 += kStreamWaves * kFusedChunk) {
        const bool two = kb0 + kStreamWaves < kb_end;     // wave-uniform: blocks kb0 and kb0 + 16
        // The previous pass's LDS accesses of these buffers are complete
        // before new loads are aimed at them.
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        float wsv[kFusedChunk];
#pragma unroll
        for (int c = 0; c < kFusedChunk; ++c) {
            const int64_t kb = kb0 + c * kStreamWaves;
            if (kb < kb_end) wsv[c] = ws_row[kb];
        }
#pragma unroll
        for (int c = 0; c < kFusedChunk; ++c) {
            const int64_t kb = kb0 + c * kStreamWaves;
            if (kb < kb_end) xrows_issue<kMp>(xrows[wave][c], rsrc_x, lane, K, kb);
        }
#pragma unroll
        for (int c = 0; c < kFusedChunk; ++c) {
            const int64_t kb = kb0 + c * kStreamWaves;
            if (kb < kb_end) slab_issue(wslab[wave][c], rsrc_w, lane_off_w, K, kb, nt_loads);
        }
        // Token rows in: the two slab loads per block issued after them may
        // still be in flight.
        if (two) wait_vmcnt<4>();
        else wait_vmcnt<2>();
        float s_r[kFusedChunk];
#pragma unroll
        for (int c = 0; c < kFusedChunk; ++c) {
            const int64_t kb = kb0 + c * kStreamWaves;
            if (kb < kb_end) {
                uint8_t* row = xrows[wave][c] + qt * kXRowStride;
                uint32_t raw[kV / 2];
                read_words<kV / 2>(row + qp * kV * 2, raw);
                float v[kV];
                float amax = 0.0f;
#pragma unroll
                for (int i = 0; i < kV / 2; ++i) {
                    v[2 * i] = kBf16 ? bf16_bits_to_float(raw[i] & 0xFFFFu) : f16_bits_to_float(raw[i] & 0xFFFFu);
                    v[2 * i + 1] = kBf16 ? bf16_bits_to_float(raw[i] >> 16) : f16_bits_to_float(raw[i] >> 16);
                    amax = fmaxf(amax, fmaxf(fabsf(v[2 * i]), fabsf(v[2 * i + 1])));
                }
                amax = token_max<kL>(amax);
                const float s = amax / 448.0f;
                uint32_t codes[(kV + 3) / 4];
                quantize_v<kV>(v, raw, s, codes);
                store_codes<kV>(row + qp * kV, codes);
                // This MFMA lane's token scale, from the first lane of token r.
                s_r[c] = token_value<kMp>(s, r_row);
            }
        }
#pragma unroll
        for (int c = 0; c < kFusedChunk; ++c) {
            const int64_t kb = kb0 + c * kStreamWaves;
            if (kb < kb_end) {
                wait_block(c, two);   // this block's weight slabs in (its weight scale is used only after this)
                u32x4 wa0, wa1;
                slab_read(wslab[wave][c], r, g, wa0, wa1);
                const uint8_t* row = xrows[wave][c] + r_row * kXRowStride;
                u32x4 b0 = *reinterpret_cast<const u32x4*>(row + 16 * g);
                u32x4 b1 = *reinterpret_cast<const u32x4*>(row + 64 + 16 * g);
                const u32x4 z4 = {0u, 0u, 0u, 0u};
                b0 = r_ok ? b0 : z4;
                b1 = r_ok ? b1 : z4;
                const i32x8 a = __builtin_bit_cast(i32x8, __builtin_shufflevector(wa0, wa1, 0, 1, 2, 3, 4, 5, 6, 7));
                const i32x8 b = __builtin_bit_cast(i32x8, __builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7));
                const f32x4 blk = mfma_e4m3_16x16x128(a, b, zero);
                const float sc = r_ok ? s_r[c] * wsv[c] : 0.0f;
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[i] = __builtin_fmaf(blk[i], sc, acc[i]);
            }
        }
    }
    __syncthreads();   // every wave is done with the slabs that red overlays
    stream_finish(acc, red, y, y_dtype, M, N, nt, 0, splits, split, n_tiles, partials, counters);
}

// ------------------------------------------------------------ wide stream ----
// All-token kernel (see w8a8_wide for where it is used): a workgroup owns
// 16 kR weight rows (kR = 1, 2 or 4 MFMA row tiles) and 16 kT tokens
// (kT = 1 for M <= 16, else 2 or 4 token tiles; grid.y covers the tokens
// beyond) over all of K,
// so no split-K hand-off is needed.  Every wave takes all kR x kT output
// tiles and the 128-K blocks w, w + W, ... (W waves: eight for kR <= 2 with
// kT <= 2, four where the slots are larger, kR = 4 or kT = 4), so each
// block's weight rows are loaded once per workgroup.  Each wave owns
// a ring of LDS slots (two or three); a slot holds one block: the
// workgroup's 16 kR weight rows, the 16 kT token rows, their token scales
// and the weight scale, brought in by direct-to-LDS loads of whole 128-byte
// lines (a load instruction covers eight full lines; register loads of MFMA
// fragments touch sixteen half lines each, which a read probe measured at
// half the throughput from L2).  A wave multiplies block j while the younger
// blocks of its ring are in flight and refills the slot as soon as it has
// read block j's operands; the slots are private, so there is no barrier
// until the end, where the W partial tiles of every output tile are summed
// in LDS in K order.  With four token tiles, eight waves of two tiles each
// (two token groups) measured slower: each group's wave loaded its own copy
// of the weight rows (4096 x 4096 M = 128 12.36 vs 11.33 us, M = 96 10.53 vs
// 10.21; 1024 x 4096 M = 512 8.34 vs 8.13); with two token tiles eight
// waves stay ahead of four (M = 24 / 32: 6.84 / 7.37 vs 7.08 / 7.52 us).
// Four weight-row tiles (a 64 x 64 output tile per wave with kT = 4) serve
// where they keep the launch to one round, e.g. 4096 x 4096 at M = 256 in
// 14.0 us against 17.7 for the best tiled plan (w8a8_wide_shape).  At long K
// on small projections the K blocks may be split over gridDim.z workgroups:
// each writes its partial tiles to the workspace and the last of a tile to
// arrive sums them in split order (the streaming kernels' hand-off).
template <int kR, int kT>
constexpr int wide_waves() { return w8a8_wide_waves(kR, kT); }
template <int kR, int kT>
struct WideSlot {
    static constexpr int kWaves = wide_waves<kR, kT>();
    static constexpr int kOffX = kR * kSlabBytes;                 // 16 kT token rows
    static constexpr int kOffXs = kOffX + kT * kSlabBytes;        // 64 token scales (lanes past 16 kT load padding)
    static constexpr int kOffWs = kOffXs + 64 * 4;                // weight scale
    static constexpr int kBytes = (kOffWs + 4 + 255) / 256 * 256;
    static constexpr int kSlotsFit = 160 * 1024 / (kWaves * kBytes);
    static constexpr int kSlots = kSlotsFit > 3 ? 3 : kSlotsFit;
    static constexpr int kVmem = 2 * kR + 2 * kT + 1 + 1;        // load instructions per block
    static_assert(kSlots >= 2, "LDS ring");
    static_assert(16 * kT <= kWave, "one token scale per lane");
};

template <int V, int Y>
__device__ __forceinline__ void wide_wait_n() {
    constexpr int n = Y * V;
    __builtin_amdgcn_s_waitcnt((n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

template <int kR, int kT>
__global__ __launch_bounds__((wide_waves<kR, kT>()) * kWave, 1) void w8a8_wide_kernel(
    const uint8_t* __restrict__ xq, const float* __restrict__ xs,
    const uint8_t* __restrict__ wq, const float* __restrict__ ws,
    void* __restrict__ y, int y_dtype, int64_t M, int64_t N, int64_t K, float* __restrict__ partials,
    uint32_t* __restrict__ counters) {
    using SL = WideSlot<kR, kT>;
    constexpr int W = SL::kWaves;
    constexpr int kWideSlots = SL::kSlots, kWideSlot = SL::kBytes;
    static_assert(kT == 1 || kT == 2 || kT == 4, "token tiles");
    static_assert(kR == 1 || kR == 2 || kR == 4, "weight-row tiles within one 128-row scale block");
    __shared__ __attribute__((aligned(1024))) uint8_t ring[W * kWideSlots * kWideSlot];
    static_assert(W * kR * kT * kWave * 16 + 16 <= W * kWideSlots * kWideSlot, "partial tiles and arrival word fit");
    const int64_t nt = blockIdx.x;            // 16 kR weight rows
    const int64_t mg = blockIdx.y;            // 16 kT tokens
    const int KB = (int)(K / 128);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave), lane = threadIdx.x % kWave;
    const int r = lane & 15, g = lane >> 4;
    const int64_t m0 = 16 * kT * mg;          // first token of the group
    const int64_t n0 = 16 * kR * nt;
    const int64_t rows_w = N - n0 < 16 * kR ? N - n0 : 16 * kR;

    const i32x4 rsrc_w = buffer_rsrc(wq + n0 * K, (uint32_t)(rows_w * K));
    // The group's token rows and their scales from row m0 on; rows at or
    // past M (and the padding scales of lanes past 16 kT) load as zeros.
    const int64_t rows_x = M - m0 > 0 ? (M - m0 < 16 * kT ? M - m0 : 16 * kT) : 0;
    const i32x4 rsrc_x = buffer_rsrc(xq + m0 * K, (uint32_t)(rows_x * K));
    const i32x4 rsrc_xs = buffer_rsrc(xs + m0 * KB, (uint32_t)(rows_x * KB * 4));
    const i32x4 rsrc_ws = buffer_rsrc(ws + (n0 / 128) * KB, (uint32_t)(KB * 4));
    const int lane_off = slab_lane_offset(lane, K);   // row lane/8, chunk (lane%8) ^ (lane/8)
    const int xs_off = lane * KB * 4;
    uint8_t* my_ring = ring + wave * kWideSlots * kWideSlot;

    auto issue = [&](int slot, int kb) {
        const uint32_t base = __builtin_amdgcn_readfirstlane(lds_address(my_ring + slot * kWideSlot));
        const int k_off = __builtin_amdgcn_readfirstlane(kb * 128);
#pragma unroll
        for (int q = 0; q < 2 * kR; ++q)
            dma16(base + 1024 * q, rsrc_w, lane_off, __builtin_amdgcn_readfirstlane((int)(8 * q * K)), k_off);
#pragma unroll
        for (int q = 0; q < 2 * kT; ++q)
            dma16(base + SL::kOffX + 1024 * q, rsrc_x, lane_off, __builtin_amdgcn_readfirstlane((int)(8 * q * K)),
                  k_off);
        dma4(base + SL::kOffXs, rsrc_xs, xs_off, __builtin_amdgcn_readfirstlane(kb * 4));
        if (lane == 0) dma4(base + SL::kOffWs, rsrc_ws, 0, __builtin_amdgcn_readfirstlane(kb * 4));
    };

    // This workgroup's K blocks: part blockIdx.z of gridDim.z.
    const int splits = (int)gridDim.z, split = (int)blockIdx.z;
    const int kb_lo = (int)((int64_t)KB * split / splits), kb_hi = (int)((int64_t)KB * (split + 1) / splits);
    const int KBs = kb_hi - kb_lo;
    const int nj = wave < KBs ? (KBs - 1 - wave) / W + 1 : 0;   // blocks of this wave
#pragma unroll
    for (int s = 0; s < kWideSlots; ++s)
        if (s < nj) issue(s, kb_lo + wave + W * s);

    f32x4 acc[kR][kT];
#pragma unroll
    for (int i = 0; i < kR; ++i)
#pragma unroll
        for (int t = 0; t < kT; ++t) acc[i][t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    const f32x4 zero = {0.0f, 0.0f, 0.0f, 0.0f};
    int slot = 0;
    for (int j = 0; j < nj; ++j) {
        // Block j is complete once at most the loads of the (up to two)
        // younger blocks are outstanding (loads retire in issue order).
        const int younger = nj - 1 - j;
        if (kWideSlots > 2 && younger >= 2) wide_wait_n<SL::kVmem, (kWideSlots > 2 ? 2 : 1)>();
        else if (younger >= 1) wide_wait_n<SL::kVmem, 1>();
        else wide_wait_n<SL::kVmem, 0>();
        asm volatile("" ::: "memory");
        const uint8_t* sl = my_ring + slot * kWideSlot;
        u32x4 a0[kR], a1[kR], b0[kT], b1[kT];
#pragma unroll
        for (int i = 0; i < kR; ++i) slab_read(sl + i * kSlabBytes, r, g, a0[i], a1[i]);
        float xsv[kT];
#pragma unroll
        for (int t = 0; t < kT; ++t) {
            slab_read(sl + SL::kOffX + t * kSlabBytes, r, g, b0[t], b1[t]);
            xsv[t] = reinterpret_cast<const float*>(sl + SL::kOffXs)[16 * t + r];
        }
        const float wsv = *reinterpret_cast<const float*>(sl + SL::kOffWs);
        // Every operand of block j is in registers before the slot is refilled.
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        if (j + kWideSlots < nj) issue(slot, kb_lo + wave + W * (j + kWideSlots));
#pragma unroll
        for (int i = 0; i < kR; ++i) {
            const i32x8 a = __builtin_bit_cast(i32x8, __builtin_shufflevector(a0[i], a1[i], 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
            for (int t = 0; t < kT; ++t) {
                const i32x8 b = __builtin_bit_cast(i32x8, __builtin_shufflevector(b0[t], b1[t], 0, 1, 2, 3, 4, 5, 6, 7));
                const f32x4 blk = mfma_e4m3_16x16x128(a, b, zero);
                const float sc = xsv[t] * wsv;
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[i][t][e] = __builtin_fmaf(blk[e], sc, acc[i][t][e]);
            }
        }
        slot = slot + 1 == kWideSlots ? 0 : slot + 1;
    }

    // Sum the W partial tiles of every output tile in K order.  Every wave's
    // loads are done (its last wait was vmcnt(0)); the barrier orders the
    // reuse of the ring.
    __syncthreads();
    float* red = reinterpret_cast<float*>(ring);
    // Slot of (row tile i, token tile t, K lane w): (((w kR + i) kT + t) * 64 + lane) * 4 floats.
#pragma unroll
    for (int i = 0; i < kR; ++i)
#pragma unroll
        for (int t = 0; t < kT; ++t)
            *reinterpret_cast<f32x4*>(red + (((wave * kR + i) * kT + t) * kWave + lane) * 4) = acc[i][t];
    __syncthreads();
    // Thread x: lane L = x % 64 of output tiles u = x / 64, x / 64 + W, ...
    // (u = i * kT + t).
    const int L = threadIdx.x % kWave, rr = L & 15, gg = L >> 4;
    auto store_tile = [&](int u, f32x4 v) {
        const int i = u / kT, tt = u % kT;
        const int64_t m = m0 + 16 * tt + rr;
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
    };
    // With K split, partial tile (tile, part, u) at float offset
    // ((tile * splits + part) * kR kT + u) * 256 + 4 L of the workspace.
    // The parts are written and read with 16-byte device-coherent (sc1)
    // buffer accesses, which go through to memory every XCD sees, as in the
    // tiled kernel's split hand-off.
    constexpr int kSc1 = 16;
    const int64_t tile = mg * (int64_t)gridDim.x + nt;
    float* tile_parts = partials == nullptr ? nullptr : partials + tile * splits * (kR * kT) * 256;
    const __amdgpu_buffer_rsrc_t prs =
        __builtin_amdgcn_make_buffer_rsrc(tile_parts, 0, splits > 1 ? splits * (kR * kT) * 256 * 4 : 0, 0x00020000);
    constexpr int kU = (kR * kT + W - 1) / W;   // output tiles per thread
    f32x4 own[kU];
#pragma unroll
    for (int iu = 0; iu < kU; ++iu) {
        const int u = (int)threadIdx.x / kWave + W * iu;
        if (u >= kR * kT) continue;
        f32x4 v = *reinterpret_cast<const f32x4*>(red + (u * kWave + L) * 4);
#pragma unroll
        for (int w = 1; w < W; ++w) v += *reinterpret_cast<const f32x4*>(red + ((w * kR * kT + u) * kWave + L) * 4);
        own[iu] = v;
        if (splits == 1)
            store_tile(u, v);
        else
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, v), prs,
                                                   ((split * (kR * kT) + u) * 256 + 4 * L) * 4, 0, kSc1);
    }
    if (splits == 1) return;
    // Hand-off as in the streaming kernels (stream_finish): every partial
    // store has completed before the barrier that precedes the counter
    // increment; the last part of the tile to arrive sums the parts in split
    // order, stores Y and re-arms the counter.
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    uint32_t* arrived = reinterpret_cast<uint32_t*>(red + W * kR * kT * kWave * 4);
    if (threadIdx.x == 0)
        *arrived = __hip_atomic_fetch_add(&counters[tile], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    if (*arrived != (uint32_t)(splits - 1)) return;
    // This workgroup's own part is still in registers (the same bits it
    // wrote): only the other parts are read back.
#pragma unroll
    for (int iu = 0; iu < kU; ++iu) {
        const int u = (int)threadIdx.x / kWave + W * iu;
        if (u >= kR * kT) continue;
        i32x4 p[4];
#pragma unroll
        for (int q = 0; q < 4; ++q)
            if (q < splits && q != split)
                p[q] = __builtin_amdgcn_raw_buffer_load_b128(prs, ((q * (kR * kT) + u) * 256 + 4 * L) * 4, 0, kSc1);
        f32x4 v = split == 0 ? own[iu] : __builtin_bit_cast(f32x4, p[0]);
#pragma unroll
        for (int q = 1; q < 4; ++q)
            if (q < splits) v += q == split ? own[iu] : __builtin_bit_cast(f32x4, p[q]);
        store_tile(u, v);
    }
    if (threadIdx.x == 0) __hip_atomic_store(&counters[tile], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

hipError_t launch_w8a8_wide(const uint8_t* xq, const float* xs, const uint8_t* wq, const float* ws,
                            void* y, int y_dtype, int64_t M, int64_t N, int64_t K, void* workspace,
                            hipStream_t stream) {
    if (M < 1 || N % 16 != 0 || K > kTileMaxK) return hipErrorInvalidValue;
    const WideShape w = w8a8_wide_shape(M, N, K);
    if (w.groups_m > 65535 || w.splits < 1 || w.splits > 4) return hipErrorInvalidValue;
    uint32_t* counters = nullptr;
    float* partials = nullptr;
    if (w.splits > 1) {
        if (!workspace) return hipErrorInvalidValue;
        counters = static_cast<uint32_t*>(workspace);
        partials = reinterpret_cast<float*>(static_cast<char*>(workspace) + w8a8_wide_counter_bytes(w));
    }
    const dim3 grid(w.groups_n, w.groups_m, (unsigned)w.splits);
#define BFP8_LAUNCH_WIDE(R, T)                                                                                   \
    hipLaunchKernelGGL((w8a8_wide_kernel<R, T>), grid, dim3(wide_waves<R, T>() * kWave), 0, stream, xq, xs, wq, ws, \
                       y, y_dtype, M, N, K, partials, counters)
    if (w.kt == 1) {
        if (w.kr == 4) BFP8_LAUNCH_WIDE(4, 1);
        else if (w.kr == 2) BFP8_LAUNCH_WIDE(2, 1);
        else BFP8_LAUNCH_WIDE(1, 1);
    } else if (w.kr == 4) {
        if (w.kt == 2) BFP8_LAUNCH_WIDE(4, 2);
        else BFP8_LAUNCH_WIDE(4, 4);
    } else if (w.kr == 1) {
        if (w.kt == 2) BFP8_LAUNCH_WIDE(1, 2);
        else BFP8_LAUNCH_WIDE(1, 4);
    } else {
        if (w.kt == 2) BFP8_LAUNCH_WIDE(2, 2);
        else BFP8_LAUNCH_WIDE(2, 4);
    }
#undef BFP8_LAUNCH_WIDE
    return hipGetLastError();
}

// ------------------------------------------------ W8A8 GEMV, M = 1 ----
// One token with K <= 16384 (batch-1 decode): the dot products run on the
// vector ALUs, laid out as in the W8A16 one-token kernel (stream_common.hpp:
// one weight row per wave, lane l covering K offsets 1024 c + 16 l of every
// 1 KB chunk c, kC chunks; the token's codes shared through LDS).  Each lane
// widens its 16 activation codes and 16 weight codes to bf16 (exact), sums
// the 16 products with v_dot2c (lane_dot16: a product of two E4M3 values is
// exact in fp32), block_sum8 gives the 128-K block's dot product to the 8
// lanes of the block, and the block is promoted once with
// xs[kb] * ws[n / 128, kb] ([ADA] "The fix"; [ARC] "What this adds").  All
// loads are issued before the first product.  gemv_row is that arithmetic;
// the kernel that quantises its own activations calls it too, so the fused
// call and quantise-then-GEMM give the same bits.
template <int kC>
__device__ __forceinline__ float gemv_row(const uint32_t (&xp)[kC][8], const float (&sx)[kC], const i32x4 (&wv)[kC],
                                          const float (&wsv)[kC]) {
    float acc = 0.0f;
#pragma unroll
    for (int c = 0; c < kC; ++c)
        acc = __builtin_fmaf(block_sum8(lane_dot16<true>(xp[c], wv[c])), sx[c] * wsv[c], acc);
    return group_sum8(acc);
}

// Issue the loads of weight row n (when `live`) and of its weight scales,
// chunk by chunk, the weights with cache policy kPol; lanes past K, and
// every lane of a row that is not live, read zeros.
template <int kC, int kPol>
__device__ __forceinline__ void gemv_load_weights(const uint8_t* wq, const float* ws, int64_t n, bool live, int64_t K,
                                                  int lane, i32x4 (&wv)[kC], float (&wsv)[kC]) {
    const int KB = (int)(K / 128);
    const int64_t nb = live ? n : 0;
    const __amdgpu_buffer_rsrc_t rw =
        __builtin_amdgcn_make_buffer_rsrc((void*)(wq + nb * K), 0, live ? (int)K : 0, 0x00020000);
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc((void*)(ws + (nb / 128) * KB), 0, live ? KB * 4 : 0, 0x00020000);
#pragma unroll
    for (int c = 0; c < kC; ++c)
        wsv[c] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, 4 * ((1024 * c + 16 * lane) / 128), 0, 0));
#pragma unroll
    for (int c = 0; c < kC; ++c) {
        const int k = 1024 * c + 16 * lane;
        wv[c] = __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(rw, k < K ? k : (int)K, 0, kPol));
    }
}

template <int kC, int kPol>
__global__ __launch_bounds__(kGemvThreads) void w8a8_gemv_kernel(
    const uint8_t* __restrict__ xq, const float* __restrict__ xs, const uint8_t* __restrict__ wq,
    const float* __restrict__ ws, void* __restrict__ y, int y_dtype, int64_t N, int64_t K) {
    constexpr int kU = (kC + 7) / 8;   // 8 KB rounds of the token's codes (1 KB per chunk)
    __shared__ __attribute__((aligned(16))) uint8_t x_lds[8192 * kU];
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave), lane = threadIdx.x % kWave;
    const int64_t n = (int64_t)blockIdx.x * kGemvWaves + wave;   // wave-uniform: scalar descriptors
    // The launch covers N exactly (N % 16 == 0); a wave past N would still
    // take part in the token copy and the barrier, reading no weights.
    const bool live = n < N;
    const int KB = (int)(K / 128);
    const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc((void*)xq, 0, (int)K, 0x00020000);
    const __amdgpu_buffer_rsrc_t rxs = __builtin_amdgcn_make_buffer_rsrc((void*)xs, 0, KB * 4, 0x00020000);
    i32x4 xr[kU], wv[kC];
    float sx[kC], wsv[kC];
    gemv_x_issue<kU>(rx, xr);
#pragma unroll
    for (int c = 0; c < kC; ++c)
        sx[c] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rxs, 4 * ((1024 * c + 16 * lane) / 128), 0, 0));
    gemv_load_weights<kC, kPol>(wq, ws, n, live, K, lane, wv, wsv);
    // Keep every load ahead of the token copy and the arithmetic: the
    // scheduler would otherwise sink the later chunks' loads below the
    // first chunk's products.
    __builtin_amdgcn_sched_barrier(0);
    gemv_x_store<kU>(x_lds, xr);
    __syncthreads();
    uint32_t xp[kC][8];
#pragma unroll
    for (int c = 0; c < kC; ++c) e4m3x16_to_bf16x2(gemv_x_read(x_lds, 64 * c + lane), xp[c]);
    const float v = gemv_row<kC>(xp, sx, wv, wsv);
    if (lane == 0 && live) store_out(y, y_dtype, n, v);
}

// The same product from 16-bit activations, quantised once per workgroup:
// kW waves, one weight row each.  The token is quantised in rounds of 4096
// values: in round t, wave w quantises activations 4096 t + (4096 / kW) w
// .. + 4096 / kW - 1, V = 4096 / (64 kW) consecutive values per lane (8 with
// eight waves), so a 1x128 group spans 128 / V lanes; their maximum (lane
// moves), scale amax / 448 and codes
// (quantize_v, the quantiser's own arithmetic) equal bfp8_quantize_act_1x128's
// bit for bit.  Codes and scales go to LDS; after one barrier every wave
// reads back its lanes' 16 codes per chunk and runs gemv_row.  The weight
// loads are issued first, so the quantisation runs while they stream.
template <bool kXBf16, int kW, int kC, int kPol>
__global__ __launch_bounds__(kW * kWave) void w8a8_gemv_quant_kernel(
    const uint16_t* __restrict__ x, const uint8_t* __restrict__ wq, const float* __restrict__ ws,
    void* __restrict__ y, int y_dtype, int64_t N, int64_t K) {
    constexpr int V = 4096 / (kW * kWave);  // activations per lane per round
    constexpr int kGroupLanes = 128 / V;
    constexpr int kRounds = kC / 4;         // 4096 values per round
    static_assert((V == 8 || V == 16) && kW * V * kWave == 4096 && kC % 4 == 0, "one round covers four chunks");
    __shared__ __attribute__((aligned(16))) uint8_t codes_lds[1024 * kC];
    __shared__ float scale_lds[8 * kC];
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave), lane = threadIdx.x % kWave;
    const int64_t n0 = (int64_t)blockIdx.x * kW + wave;    // wave-uniform; < N since kW divides N

    // This wave's share of the activations first (values past K load as
    // zeros: their groups get scale 0 and code 0), then its weight row: loads
    // complete in issue order, so the quantisation waits only for the former.
    const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc((void*)x, 0, (int)(2 * K), 0x00020000);
    uint32_t raw[kRounds][V / 2];
#pragma unroll
    for (int t = 0; t < kRounds; ++t) {
        const int i0 = 4096 * t + (4096 / kW) * wave + V * lane;
#pragma unroll
        for (int h = 0; h < V / 8; ++h) {
            const i32x4 u = __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, 2 * i0 + 16 * h, 0, 0));
#pragma unroll
            for (int j = 0; j < 4; ++j) raw[t][4 * h + j] = (uint32_t)u[j];
        }
    }
    // Every wave's activation loads go out before any wave's weight loads
    // (a bare barrier: it waits for no load), so the activations do not
    // queue behind the weights in the memory system.
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    i32x4 wv[kC];
    float wsv[kC];
    gemv_load_weights<kC, kPol>(wq, ws, n0, true, K, lane, wv, wsv);
    __builtin_amdgcn_sched_barrier(0);   // keep the weight loads ahead of the quantisation

#pragma unroll
    for (int t = 0; t < kRounds; ++t) {
        const int i0 = 4096 * t + (4096 / kW) * wave + V * lane;
        float v[V];
#pragma unroll
        for (int j = 0; j < V / 2; ++j) {
            v[2 * j] = kXBf16 ? bf16_bits_to_float(raw[t][j] & 0xFFFFu) : f16_bits_to_float(raw[t][j] & 0xFFFFu);
            v[2 * j + 1] = kXBf16 ? bf16_bits_to_float(raw[t][j] >> 16) : f16_bits_to_float(raw[t][j] >> 16);
        }
        float amax = 0.0f;
#pragma unroll
        for (int j = 0; j < V; ++j) amax = fmaxf(amax, fabsf(v[j]));
        amax = group_max<kGroupLanes>(amax);
        const float s = amax / 448.0f;
        uint32_t q[V / 4];
        quantize_v<V>(v, raw[t], s, q);
#pragma unroll
        for (int j = 0; j < V / 4; ++j) reinterpret_cast<uint32_t*>(codes_lds + i0)[j] = q[j];
        if (lane % kGroupLanes == 0) scale_lds[i0 / 128] = s;
    }
    __syncthreads();

    uint32_t xp[kC][8];
    float sx[kC];
#pragma unroll
    for (int c = 0; c < kC; ++c) {
        const int k = 1024 * c + 16 * lane;
        e4m3x16_to_bf16x2(*reinterpret_cast<const i32x4*>(codes_lds + k), xp[c]);
        // Lanes past K: their weights are zero; take scale 0 so that no
        // stale value enters the promotion.
        sx[c] = k < K ? scale_lds[k / 128] : 0.0f;
    }
    const float v = gemv_row<kC>(xp, sx, wv, wsv);
    if (lane == 0) store_out(y, y_dtype, n0, v);
}

hipError_t launch_w8a8_gemv(const uint8_t* xq, const float* xs, const uint8_t* wq, const float* ws, void* y,
                            int y_dtype, int64_t N, int64_t K, hipStream_t stream) {
    if (N % 16 != 0 || K > kGemvMaxK) return hipErrorInvalidValue;
    static_assert(kGemvWaves == kGemvLaunchWaves, "plan and launch agree");
    const dim3 grid((unsigned)((N + kGemvWaves - 1) / kGemvWaves));
#define BFP8_LAUNCH_GEMV8(C, P)                                                                                   \
    hipLaunchKernelGGL((w8a8_gemv_kernel<C, P>), grid, dim3(kGemvThreads), 0, stream, xq, xs, wq, ws, y, y_dtype, N, K)
#define BFP8_LAUNCH_GEMV8_C(P)                    \
    switch (gemv_chunks(K)) {                      \
        case 4: BFP8_LAUNCH_GEMV8(4, P); break;   \
        case 8: BFP8_LAUNCH_GEMV8(8, P); break;   \
        case 12: BFP8_LAUNCH_GEMV8(12, P); break; \
        default: BFP8_LAUNCH_GEMV8(16, P); break; \
    }
    if (weights_nt(N, K)) { BFP8_LAUNCH_GEMV8_C(kLoadNt) }
    else { BFP8_LAUNCH_GEMV8_C(0) }
#undef BFP8_LAUNCH_GEMV8_C
#undef BFP8_LAUNCH_GEMV8
    return hipGetLastError();
}

hipError_t launch_w8a8_gemv_quant(const void* x, bool x_bf16, const uint8_t* wq, const float* ws, void* y,
                                  int y_dtype, int64_t N, int64_t K, hipStream_t stream) {
    if (N % 16 != 0 || K > kGemvMaxK) return hipErrorInvalidValue;   // every wave owns a row
    const uint16_t* xh = static_cast<const uint16_t*>(x);
    // Eight waves (rows) per workgroup: each wave quantises an eighth of each
    // 4096 values, 8 values per lane, its group maximum all in lane moves.
    // Every workgroup quantises the whole token, so fewer, larger workgroups
    // do less of that work in all: N = K = 4096, 5.0-5.06 us against
    // 5.25-5.29 for four waves (16 values per lane) and 5.43 for sixteen.
    constexpr int kQW = kGemvWaves;
    const dim3 grid((unsigned)(N / kQW));
#define BFP8_LAUNCH_GEMVQ(B, C, P)                                                                                 \
    hipLaunchKernelGGL((w8a8_gemv_quant_kernel<B, kQW, C, P>), grid, dim3(kQW * kWave), 0, stream, xh, wq, ws, y,      \
                       y_dtype, N, K)
#define BFP8_LAUNCH_GEMVQ_C(B, P)                    \
    switch (gemv_chunks(K)) {                         \
        case 4: BFP8_LAUNCH_GEMVQ(B, 4, P); break;   \
        case 8: BFP8_LAUNCH_GEMVQ(B, 8, P); break;   \
        case 12: BFP8_LAUNCH_GEMVQ(B, 12, P); break; \
        default: BFP8_LAUNCH_GEMVQ(B, 16, P); break; \
    }
    const bool nt = weights_nt(N, K);
    if (x_bf16) {
        if (nt) { BFP8_LAUNCH_GEMVQ_C(true, kLoadNt) }
        else { BFP8_LAUNCH_GEMVQ_C(true, 0) }
    } else {
        if (nt) { BFP8_LAUNCH_GEMVQ_C(false, kLoadNt) }
        else { BFP8_LAUNCH_GEMVQ_C(false, 0) }
    }
#undef BFP8_LAUNCH_GEMVQ_C
#undef BFP8_LAUNCH_GEMVQ
    return hipGetLastError();
}

hipError_t launch_w8a8_stream(const uint8_t* xq, const float* xs, const uint8_t* wq, const float* ws,
                              void* y, int y_dtype, int64_t M, int64_t N, int64_t K,
                              void* workspace, hipStream_t stream) {
    const StreamPlan p = plan_stream(M, N, K);
    if (p.m_tiles > 65535) return hipErrorInvalidValue;
    uint32_t* counters;
    float* partials;
    if (!stream_workspace_parts(p, workspace, counters, partials)) return hipErrorInvalidValue;
    const dim3 grid((unsigned)p.n_tiles, (unsigned)p.splits, (unsigned)p.m_tiles);   // one 16-token tile per z
    {
#define BFP8_LAUNCH_LDS(MP)                                                                                    \
    hipLaunchKernelGGL(w8a8_stream_lds_kernel<MP>, grid, dim3(kStreamThreads), 0, stream, xq, xs, wq, ws, y, y_dtype, \
                       M, N, K, p.n_tiles, p.splits, p.kb_per_split, partials, counters)
        switch (M <= 1 ? 1 : M <= 2 ? 2 : M <= 4 ? 4 : M <= 8 ? 8 : 16) {
            case 1: BFP8_LAUNCH_LDS(1); break;
            case 2: BFP8_LAUNCH_LDS(2); break;
            case 4: BFP8_LAUNCH_LDS(4); break;
            case 8: BFP8_LAUNCH_LDS(8); break;
            default: BFP8_LAUNCH_LDS(16); break;
        }
#undef BFP8_LAUNCH_LDS
    }
    return hipGetLastError();
}

template <bool kBf16>
static void launch_quant_mp(int mp, dim3 grid, hipStream_t stream, const void* x, const uint8_t* wq, const float* ws,
                            void* y, int y_dtype, int64_t M, int64_t N, int64_t K, const StreamPlan& p,
                            float* partials, uint32_t* counters) {
    const uint16_t* xh = static_cast<const uint16_t*>(x);
#define BFP8_LAUNCH_MP(MP)                                                                                    \
    hipLaunchKernelGGL((w8a8_stream_quant_kernel<kBf16, MP>), grid, dim3(kStreamThreads), 0, stream, xh, wq, ws, \
                       y, y_dtype, M, N, K, p.n_tiles, p.splits, p.kb_per_split, partials, counters)
    switch (mp) {
        case 1: BFP8_LAUNCH_MP(1); break;
        case 2: BFP8_LAUNCH_MP(2); break;
        case 4: BFP8_LAUNCH_MP(4); break;
        default: BFP8_LAUNCH_MP(8); break;
    }
#undef BFP8_LAUNCH_MP
}

hipError_t launch_w8a8_stream_quant(const void* x, bool x_bf16, const uint8_t* wq, const float* ws,
                                    void* y, int y_dtype, int64_t M, int64_t N, int64_t K,
                                    void* workspace, hipStream_t stream) {
    const StreamPlan p = plan_stream(M, N, K);
    uint32_t* counters;
    float* partials;
    if (!stream_workspace_parts(p, workspace, counters, partials)) return hipErrorInvalidValue;
    const dim3 grid((unsigned)p.n_tiles, (unsigned)p.splits, 1u);
    const int mp = M <= 1 ? 1 : M <= 2 ? 2 : M <= 4 ? 4 : 8;
    if (x_bf16) {
        launch_quant_mp<true>(mp, grid, stream, x, wq, ws, y, y_dtype, M, N, K, p, partials, counters);
    } else {
        launch_quant_mp<false>(mp, grid, stream, x, wq, ws, y, y_dtype, M, N, K, p, partials, counters);
    }
    return hipGetLastError();
}

}  // namespace bfp8
