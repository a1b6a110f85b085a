// W8A8 blockwise GEMM, tiled kernels for M > 16 on gfx950; the same kernel
// serves the weight-only products at larger M (TileX: 16-bit token rows,
// E4M3 weights widened in registers, with 128x128 fp32 weight scales or
// block-32 UE8M0 scales applied in the widening).
//
// A workgroup computes a BN (weight rows n) x BM (tokens m) tile of Y over a
// range of 128-wide K blocks, one scale block per LDS stage ([ARC] "What
// this adds": the K tile is the scale block, so each stage has one scale per
// row block and token).  Eight waves, two per SIMD, tile the workgroup tile;
// two waves per SIMD let one wave's promotion FMAs run in the shadow of the
// other wave's MFMAs, and each wave's fp32 accumulators, operand fragments
// and block temporaries fit its 256 registers without spilling ([ADA]
// "Where the registers went").
//
// Per 128-K block and 16x16 tile: one FP8 MFMA 16x16x128 with a zero
// accumulator gives the block partial P, and one fp32 FMA per output applies
// xs[m, kb] * ws[n/128, kb] ([ADA] "The fix").  Weight rows are the MFMA row
// operand and tokens the column operand, so every lane's four outputs share
// one token and one weight-scale row: one combined scale per lane per tile
// column per block.
//
// Data movement: global -> LDS with direct-to-LDS 16-byte buffer loads
// (buffer_load_dwordx4 ... lds; the lane at LDS granule p fetches whichever
// global 16 bytes belong there), two or three LDS stages, one barrier per
// block.  LDS rows are 128 bytes (eight 16-byte chunks); chunk c of row r is
// stored at chunk position c ^ (r & 7), which makes the MFMA fragment reads
// (16 rows, same chunk) conflict-free.  Fragment K order: MFMA K slot g
// (lanes 16g..16g+15) takes chunks g and g + 4 of the row, the same for both
// operands, so the contraction is over the same 128 K values.
//
// Tile shapes ([ADA] "One tile doesn't fit all M"): 256x256, 256x128,
// 128x128, 64x128 and 128x64, the last three with K optionally split over
// several workgroups; plan_tile picks the shape and split with the least
// estimated time (a cost model fitted to measured per-block and hand-off
// times).  Split partial tiles go to the
// workspace in fp32 and the last workgroup of a tile sums them in split
// order (no float atomics, identical from run to run), with the same
// fence-free hand-off as the streaming kernels.

#include <type_traits>

#include "bfp8_device.hpp"
#include "bfp8_launch.hpp"

namespace bfp8 {

namespace {


constexpr int kRowBytes = 128;                          // one 128-K block of one row
constexpr int kRowsPerLoad = kWave * 16 / kRowBytes;    // 8 rows per 16-byte load instruction
constexpr int kCUs = 256;

// Token operand of a tile configuration: E4M3 codes with 1x128 scales
// (W8A8), or 16-bit activations with E4M3 weights widened in registers
// (W8A16, bf16 or fp16, 128x128 fp32 weight scales; or fp16 with block-32
// UE8M0 weight scales, kTileF16Blk32).
enum TileX { kTileCodes = 0, kTileBf16 = 1, kTileF16 = 2, kTileF16Blk32 = 3 };

template <int BN_, int BM_, int WAVES_N, int WAVES_M, bool SPLIT, int X_ = kTileCodes, int FILL_ROWS_ = 0>
struct TileCfg {
    static constexpr int BN = BN_, BM = BM_;
    static constexpr int X = X_;
    static constexpr bool kX16 = X_ != kTileCodes;  // 16-bit token rows, no token scales
    static constexpr bool kXBf16 = X_ == kTileBf16;
    // Block-32 weights: the stage's per-wave scale word holds the four UE8M0
    // bytes of the block's 32x32 tiles in the wave's 32-row band, applied
    // in the widening, and the MFMAs accumulate across K with no promotion.
    static constexpr bool kBlk32 = X_ == kTileF16Blk32;
    static constexpr bool kSplit = SPLIT;           // plans for this shape may split K
    static constexpr int kWavesN = WAVES_N, kWavesM = WAVES_M;
    static constexpr int kWaves = kWavesN * kWavesM;
    static constexpr int kThreads = kWaves * kWave;
    static constexpr int kWaveN = BN / kWavesN, kWaveM = BM / kWavesM;   // per-wave tile
    static constexpr int kTi = kWaveN / 16, kTj = kWaveM / 16;
    static constexpr int kBRowBytes = kX16 ? 256 : kRowBytes;           // token row bytes per 128-K block
    static constexpr int kBRowsPerLoad = kWave * 16 / kBRowBytes;       // token rows per load instruction
    static constexpr int kStageA = BN * kRowBytes;
    static constexpr int kStageB = BM * kBRowBytes;
    static constexpr int kLoadsA = BN / (kRowsPerLoad * kWaves);        // weight-row loads per wave per stage
    static constexpr int kLoadsPerWave = kLoadsA + BM / (kBRowsPerLoad * kWaves);
    static constexpr int kXsLanes = kX16 ? 0 : BM / kWaves;             // token scales per wave
    static constexpr int kOffXs = kStageA + kStageB;
    static constexpr int kOffWs = kOffXs + (kX16 ? 0 : BM * 4);
    static constexpr int kStageBytes = kOffWs + kWaves * 4;
    static constexpr int kStageStride = (kStageBytes + 1023) / 1024 * 1024;
    // As many LDS stages as fit, up to six: blocks kb+1 .. kb+S-1 are in
    // flight while block kb is multiplied.  The small tiles are bound by
    // memory latency rather than by the matrix core, so they need the deep
    // prefetch to keep enough bytes in flight per CU.
    static constexpr int kStages = (160 * 1024 - 256) / kStageStride < 6 ? (160 * 1024 - 256) / kStageStride : 6;
    // Vector-memory instructions one stage adds per wave: tile loads, the
    // token scales (W8A8 only) and the weight scale.
    static constexpr int kVmemPerStage = kLoadsPerWave + (kX16 ? 1 : 2);
    // The refill loads of a block are spread over its first kFillRows MFMA
    // rows (row i issues tile loads fill_lo(i) .. fill_lo(i + 1) - 1).
    static constexpr int kFillRows = FILL_ROWS_ > 0 && FILL_ROWS_ < kTi ? FILL_ROWS_ : kTi;
    static constexpr int fill_lo(int i) { return (i < kFillRows ? i : kFillRows) * kLoadsPerWave / kFillRows; }
    // W8A16 with many token tiles per wave: token fragments are streamed one
    // tile column at a time (all of them would not fit in registers) and the
    // widened weight rows are kept for the whole block.
    static constexpr bool kJOuter = kX16 && kTj > 4;
    static constexpr int kFillCols = kTj / 2;   // j-outer: refill loads over the first half of the columns
    static constexpr int fill_lo_j(int j) { return (j < kFillCols ? j : kFillCols) * kLoadsPerWave / kFillCols; }
    static_assert(kStages * kStageStride <= 160 * 1024, "LDS budget");
    static_assert(BN % (kRowsPerLoad * kWaves) == 0 && BM % (kBRowsPerLoad * kWaves) == 0, "load split");
    static_assert(kX16 || (kXsLanes >= 1 && kXsLanes <= kWave), "token-scale loads");
    static_assert(128 % kWaveN == 0 || kWaveN % 128 == 0, "one weight-scale row per wave");
    static_assert(!kBlk32 || kWaveN == 32, "one 32-row scale band per wave");
    static_assert(kTi >= 1 && kTj >= 1 && kStages >= 2 && (kStages - 2) * kVmemPerStage < 64, "wave tile");
};

// With two stages the next block's loads have only the current block's
// compute to land in: they are issued over its first four MFMA rows (of
// eight), not all eight, so the last of them is not issued just before the
// wait at the top of the next block (3% at M = N = K = 4096, random data).
using Cfg256 = TileCfg<256, 256, 2, 4, false, kTileCodes, 4>;    // wave tile 128 n x 64 m, 2 stages
using Cfg128 = TileCfg<128, 128, 2, 4, true>;     // 64 x 32, 4 stages
using Cfg256x128 = TileCfg<256, 128, 4, 2, false>;   // 64 x 64, 3 stages
using Cfg64x128 = TileCfg<64, 128, 2, 4, true>;   // 32 x 32, 6 stages
using Cfg128x64 = TileCfg<128, 64, 4, 2, true>;   // 32 x 32, 6 stages
// W8A16 (16-bit activations): wave tiles 32 x 64 and 32 x 32 (four waves
// across the weight rows, so each decoded weight fragment feeds kTj MFMAs).
template <int X> using Cfg16_128 = TileCfg<128, 128, 4, 2, true, X>;   // 3 stages
template <int X> using Cfg16_64 = TileCfg<128, 64, 4, 2, true, X>;     // 4 stages
// Large M: 256 weight rows x 128 tokens, eight waves stacked along the
// weight rows (wave tile 32 x 128), so each widened weight fragment feeds
// eight token tiles; two stages.
template <int X> using Cfg16_256 = TileCfg<256, 128, 8, 1, false, X>;

// s_waitcnt vmcnt(N) lgkmcnt(0) (expcnt not waited for).
template <int N>
__device__ __forceinline__ void wait_vm_lgkm0() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4));
}

// Wait until at most `younger` stages of this wave's loads are outstanding
// (each stage is C::kVmemPerStage instructions and loads retire in issue
// order), and for all of its LDS reads.
template <class C, int Y = C::kStages - 2>
__device__ __forceinline__ void wait_stage(int younger) {
    if constexpr (Y == 0) {
        wait_vm_lgkm0<0>();
    } else {
        if (younger >= Y) wait_vm_lgkm0<Y * C::kVmemPerStage>();
        else wait_stage<C, Y - 1>(younger);
    }
}

// LDS swizzles: chunk c of stage row R sits at chunk position c ^ s(R).
// Token rows are read 16 consecutive rows at a time, so s_B(R) = R & 7.
// Weight rows are read in the permuted order of a_row() below (groups of
// four consecutive rows, 8 rows apart), so s_A mixes bits 1, 3 and 4 of the
// row.  Either way the 16 lanes of one ds_read_b128 phase hit 16 distinct
// 16-byte bank groups.
__device__ __forceinline__ int swz_a_bits(int row) { return ((row >> 1) & 1) | (((row >> 3) & 3) << 1); }
__device__ __forceinline__ int swz_a(int row, int c) { return row * kRowBytes + ((c ^ swz_a_bits(row)) << 4); }
__device__ __forceinline__ int swz_b(int row, int c) { return row * kRowBytes + ((c ^ (row & 7)) << 4); }
// 16-bit token rows are 256 bytes (16 chunks) per block: chunk c of row R at
// position c ^ (R & 15), so 16 consecutive rows read at one chunk hit 16
// distinct bank groups.
__device__ __forceinline__ int swz_b16(int row, int c) { return row * 256 + ((c ^ (row & 15)) << 4); }

// Weight row (local to the wave's kWaveN rows) behind MFMA row rho of the
// wave's weight tile i.  Chosen so that the MFMA output lane group g (rows
// 4g..4g+3 of every tile) holds, over tile pairs (2p, 2p+1), the eight
// consecutive rows 32p + 8g .. 32p + 8g + 7: each lane then stores 16
// contiguous bytes per pair, and the four lane groups 64 contiguous bytes.
__device__ __forceinline__ int a_row(int i, int rho) {
    return 32 * (i >> 1) + 4 * (i & 1) + 8 * (rho >> 2) + (rho & 3);
}

// Issue this wave's direct-to-LDS loads of K block kb into a stage.
// Instruction q of wave w fills LDS rows 8*(W q + w) .. +7 of the stage (W =
// waves; weight rows first, then token rows); lane l fills granule l of those
// 1 KB, i.e. row R = 8*(W q + w) + l/8 at chunk position l%8, so it
// fetches logical chunk (l%8) ^ s(R) of that row (s_A or s_B; with W a
// multiple of 4 both are the same for every q, so one lane offset per
// operand serves all q).  The row offset goes into the
// per-lane offset, which the descriptor's range check sees, so rows past the
// end of the matrix load as zeros; the K block's byte offset (< K, so it
// never carries a valid row's access past its own row) goes into the scalar
// offset.
// Only tile loads q_lo <= q < q_hi are issued, and the two scale loads only
// with `scales` (the caller spreads one stage's loads over its MFMA rows).
//
// 16-bit token rows (W8A16) are 256 bytes per block: a load instruction then
// covers 4 rows (lane l: row 4*(W q + w) + l/16, chunk position l%16), and
// the K block's offset in them is kb * 256.
template <class C>
__device__ __forceinline__ void issue_stage(uint8_t* stage, i32x4 rsrc_a, i32x4 rsrc_b, i32x4 rsrc_xs,
                                            i32x4 rsrc_ws, int lane_off_a, int lane_off_b, int q_stride,
                                            int q_stride_b, int xs_off, int64_t kb, int wave, int lane,
                                            int q_lo = 0, int q_hi = C::kLoadsPerWave, bool scales = true) {
    const int k_off = __builtin_amdgcn_readfirstlane((int)(kb * kRowBytes));
    const int k_off_b = __builtin_amdgcn_readfirstlane((int)(kb * C::kBRowBytes));
    const uint32_t base = lds_address(stage);
    if (scales) {
        // Token scales xs[m0 + kXsLanes * w + l, kb], lanes l < kXsLanes only
        // (the dword form writes M0 + 4 * lane for every active lane).
        if (!C::kX16 && lane < C::kXsLanes)
            dma4(__builtin_amdgcn_readfirstlane(base + C::kOffXs + 4 * C::kXsLanes * wave), rsrc_xs, xs_off,
                 __builtin_amdgcn_readfirstlane((int)(kb * 4)));
        // This wave's weight scale ws[nb, kb], lane 0 only.
        if (lane == 0)
            dma4(__builtin_amdgcn_readfirstlane(base + C::kOffWs + 4 * wave), rsrc_ws, 0,
                 __builtin_amdgcn_readfirstlane((int)(kb * 4)));
    }
#pragma unroll
    for (int q = 0; q < C::kLoadsPerWave; ++q) {
        if (q < q_lo || q >= q_hi) continue;
        const uint32_t lds = __builtin_amdgcn_readfirstlane(base + kRowsPerLoad * (C::kWaves * q + wave) * kRowBytes);
        if (q < C::kLoadsA) {
            dma16(lds, rsrc_a, lane_off_a, __builtin_amdgcn_readfirstlane(q * q_stride), k_off);
        } else {
            dma16(lds, rsrc_b, lane_off_b, __builtin_amdgcn_readfirstlane((q - C::kLoadsA) * q_stride_b), k_off_b);
        }
    }
}

// Workgroup barrier without the memory fence of __syncthreads(): that fence
// would wait for every outstanding direct-to-LDS load, including the
// prefetch of the next stages.  Visibility is handled by explicit counter
// waits instead (own stage loads complete before the barrier; own LDS reads
// complete before the barrier that frees a stage for reuse); the empty asm
// statements keep the compiler from moving memory accesses across it.
__device__ __forceinline__ void stage_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

template <bool kWeightRows>
__device__ __forceinline__ i32x8 read_frag(const uint8_t* stage, int row, int g) {
    const int lo_off = kWeightRows ? swz_a(row, g) : swz_b(row, g);
    const int hi_off = kWeightRows ? swz_a(row, g + 4) : swz_b(row, g + 4);
    const u32x4 lo = *reinterpret_cast<const u32x4*>(stage + lo_off);
    const u32x4 hi = *reinterpret_cast<const u32x4*>(stage + hi_off);
    return __builtin_bit_cast(i32x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Workgroup -> (tile, split).  Workgroups are dealt round-robin to the 8
// XCDs; each XCD gets a contiguous run of indices, in which the splits of a
// tile are adjacent and tiles come in groups of up to 8 token tiles per
// weight tile, so the workgroups resident on one XCD share weight and token
// rows in that XCD's L2.
__device__ __forceinline__ void tile_of_block(int64_t b, int64_t tiles_n, int64_t tiles_m, int64_t splits,
                                              int64_t& t, int64_t& split, int64_t& tn, int64_t& tm) {
    const int64_t total = tiles_n * tiles_m * splits;
    if (total % 8 == 0) b = (b % 8) * (total / 8) + b / 8;
    split = b % splits;
    t = b / splits;
    constexpr int64_t kGroup = 8;
    const int64_t per_group = kGroup * tiles_n;
    const int64_t group = t / per_group;
    const int64_t first_m = group * kGroup;
    const int64_t group_m = tiles_m - first_m < kGroup ? tiles_m - first_m : kGroup;
    const int64_t in_group = t - group * per_group;
    tm = first_m + in_group % group_m;
    tn = in_group / group_m;
}

// Store eight consecutive outputs y[idx .. idx+7] (lo = the first four):
// one 16-byte store for 16-bit outputs, two for fp32.  idx is a multiple of
// 8 and, with N % 16 == 0, the eight lie in one row.  Non-temporal stores:
// the output is not read again by this kernel, and with every workgroup of
// a one-round grid storing at the same time the streaming hint measured 2 %
// faster at M = N = K = 4096 (69.8 -> 68.4 us; a store through LDS in whole
// 128-byte lines measured no faster than these 64-byte row pieces).
__device__ __forceinline__ void store8(void* y, int y_dtype, int64_t idx, f32x4 lo, f32x4 hi) {
    if (y_dtype == 2) {
        __builtin_nontemporal_store(lo, reinterpret_cast<f32x4*>(static_cast<float*>(y) + idx));
        __builtin_nontemporal_store(hi, reinterpret_cast<f32x4*>(static_cast<float*>(y) + idx + 4));
    } else {
        uint32_t h[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            h[e] = y_dtype == 0 ? float_to_bf16_bits(lo[e]) : float_to_f16_bits(lo[e]);
            h[e + 4] = y_dtype == 0 ? float_to_bf16_bits(hi[e]) : float_to_f16_bits(hi[e]);
        }
        __builtin_nontemporal_store(
            u32x4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)},
            reinterpret_cast<u32x4*>(static_cast<uint16_t*>(y) + idx));
    }
}

}  // namespace

// Grid: tiles_n * tiles_m * splits workgroups.  Split s of a tile covers K
// blocks [s * kb_per_split, min(KB, (s + 1) * kb_per_split)).  With splits
// > 1, `partials` holds splits fp32 BN x BM tiles per output tile and
// `counters` one uint32 per output tile (zero on entry, re-armed on exit).
template <class C>
__global__ __launch_bounds__(C::kThreads, 1) void w8a8_tile_kernel(
    const void* __restrict__ xin, const float* __restrict__ xs,
    const uint8_t* __restrict__ wq, const void* __restrict__ wscale,
    void* __restrict__ y, int y_dtype, int64_t M, int64_t N, int64_t K,
    int64_t tiles_n, int64_t tiles_m, int64_t splits, int64_t kb_per_split,
    float* __restrict__ partials, uint32_t* __restrict__ counters) {
    __shared__ __attribute__((aligned(1024))) uint8_t stages[C::kStages * C::kStageStride];
    __shared__ uint32_t arrived;

    int64_t t, split, tn, tm;
    tile_of_block(blockIdx.x, tiles_n, tiles_m, splits, t, split, tn, tm);
    const int64_t n0 = tn * C::BN, m0 = tm * C::BM;
    const int64_t KB = K / 128, NB = (N + 127) / 128;
    const int64_t kb0 = split * kb_per_split;
    const int64_t nkb = KB - kb0 < kb_per_split ? KB - kb0 : kb_per_split;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave), lane = threadIdx.x % kWave;
    const int wn = wave % C::kWavesN, wm = wave / C::kWavesN;
    const int r = lane & 15, g = lane >> 4;

    // Buffer descriptors over this workgroup's weight rows, token rows and
    // token-scale rows; rows past N or M lie outside them and load as zeros.
    const int64_t rows_a = N - n0 < C::BN ? N - n0 : C::BN;
    const int64_t rows_b = M - m0 < C::BM ? M - m0 : C::BM;
    // Token operand: E4M3 codes (1 byte) or 16-bit activations (2 bytes).
    constexpr int64_t kXBytes = C::kX16 ? 2 : 1;
    const uint8_t* xbase = static_cast<const uint8_t*>(xin);
    const i32x4 rsrc_a = buffer_rsrc(wq + n0 * K, (uint32_t)(rows_a * K));
    const i32x4 rsrc_b = buffer_rsrc(xbase + m0 * K * kXBytes, (uint32_t)(rows_b * K * kXBytes));
    const i32x4 rsrc_xs = C::kX16 ? rsrc_b : buffer_rsrc(xs + m0 * KB, (uint32_t)(rows_b * KB * 4));
    const int dma_row = 8 * wave + (lane >> 3);     // stage row of this lane's first load, minus 8 W q
    const int lane_off_a = (int)(dma_row * K) + (((lane & 7) ^ swz_a_bits(dma_row)) << 4);
    int lane_off_b;
    if constexpr (C::kX16) {
        const int row16 = 4 * wave + (lane >> 4);   // 16-bit token row of this lane's first load
        lane_off_b = (int)(row16 * K * 2) + (((lane & 15) ^ (row16 & 15)) << 4);
    } else {
        lane_off_b = (int)(dma_row * K) + (((lane & 7) ^ (dma_row & 7)) << 4);
    }
    const int q_stride = (int)(kRowsPerLoad * C::kWaves * K);
    const int q_stride_b = (int)(C::kBRowsPerLoad * C::kWaves * K * kXBytes);
    const int xs_off = (int)((C::kXsLanes * wave + lane) * KB * 4);

    // Weight scales: one row of ws per wave (its weight rows share it), or
    // for block-32 the wave's 32-row band of UE8M0 bytes (K / 32 a band, a
    // dword of four per 128-K block).  A wave whose rows lie past N takes
    // the last row or band, so its scale loads stay inside the array.
    const i32x4 rsrc_ws = [&] {
        if constexpr (C::kBlk32) {
            int64_t band = (n0 + C::kWaveN * wn) / 32;
            band = band < N / 32 ? band : N / 32 - 1;
            return buffer_rsrc(static_cast<const uint8_t*>(wscale) + band * (K / 32), (uint32_t)(KB * 4));
        } else {
            int64_t nb = (n0 + C::kWaveN * wn) / 128;
            nb = nb < NB ? nb : NB - 1;
            return buffer_rsrc(static_cast<const float*>(wscale) + nb * KB, (uint32_t)(KB * 4));
        }
    }();
    // Block-32: this lane's two UE8M0 scales of a block (chunk g, K 16 g ..
    // 16 g + 15, lies in tile 4 kb + g / 2; chunk g + 4 in tile
    // 4 kb + 2 + g / 2) from the stage's scale word.
    auto band_scales = [&](const uint8_t* stage, float& e0, float& e1) {
        const uint32_t sw = reinterpret_cast<const uint32_t*>(stage + C::kOffWs)[wave];
        e0 = ue8m0_scale((sw >> (8 * (g >> 1))) & 0xFF);
        e1 = ue8m0_scale((sw >> (8 * (2 + (g >> 1)))) & 0xFF);
    };

    f32x4 acc[C::kTi][C::kTj];
#pragma unroll
    for (int i = 0; i < C::kTi; ++i)
#pragma unroll
        for (int j = 0; j < C::kTj; ++j) acc[i][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    const f32x4 zero = {0.0f, 0.0f, 0.0f, 0.0f};

    const int a_base = C::kWaveN * wn;               // + a_row(i, r)
    const int b_row0 = C::BN + C::kWaveM * wm + r;   // + 16 j

    // Per block, per wave: kTi rows of kTj MFMAs (one per 16x16 tile) into
    // block temporaries; the FMAs that promote row i are issued after row
    // i+1's MFMAs, so the matrix core and the VALU work on different rows.
    // The token fragments and the scales of the block are read first; the
    // weight fragments are streamed one row ahead.
    // `fill` (when not null) is the stage that receives block fill_kb; its
    // loads are issued between the MFMA rows, so a wave never waits for the
    // memory pipeline to accept a whole stage before it starts multiplying.
    auto compute = [&](const uint8_t* stage, auto refill, uint8_t* fill, int64_t fill_kb) {
      if constexpr (C::kJOuter) {
        // The kTi weight rows of the block are widened once (aop), then each
        // token tile column j is read (one ahead) and multiplied by every row;
        // the promotion of column j - 1 follows the MFMAs of column j.
        const float wsc = reinterpret_cast<const float*>(stage + C::kOffWs)[wave];
        float e0 = 1.0f, e1 = 1.0f;
        if constexpr (C::kBlk32) band_scales(stage, e0, e1);
        u32x4 aop[C::kTi][4];
#pragma unroll
        for (int i = 0; i < C::kTi; ++i) {
            const i32x8 af = read_frag<true>(stage, a_base + a_row(i, r), g);
#pragma unroll
            for (int jj = 0; jj < 4; ++jj)
                aop[i][jj] = widen8<C::kXBf16>((uint32_t)af[2 * jj], (uint32_t)af[2 * jj + 1], jj < 2 ? e0 : e1);
        }
        auto read_b = [&](int j, u32x4 (&b)[4]) {
            const int row = C::kWaveM * wm + 16 * j + r;
#pragma unroll
            for (int jj = 0; jj < 4; ++jj)
                b[jj] = *reinterpret_cast<const u32x4*>(stage + C::kStageA +
                                                        swz_b16(row, 2 * g + 8 * (jj >> 1) + (jj & 1)));
        };
        u32x4 bcur[4], bnext[4];
        read_b(0, bcur);
        f32x4 tmp[2][C::kTi];
#pragma unroll
        for (int j = 0; j < C::kTj; ++j) {
            const int c = j & 1;
            if (j + 1 < C::kTj) read_b(j + 1, bnext);
#pragma unroll
            for (int i = 0; i < C::kTi; ++i) {
                if constexpr (C::kBlk32) {
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) acc[i][j] = mfma_f16_16x16x32(aop[i][jj], bcur[jj], acc[i][j]);
                } else {
                    f32x4 blk = zero;
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj)
                        blk = C::kXBf16 ? mfma_bf16_16x16x32(aop[i][jj], bcur[jj], blk)
                                        : mfma_f16_16x16x32(aop[i][jj], bcur[jj], blk);
                    tmp[c][i] = blk;
                }
            }
            if constexpr (decltype(refill)::value)
                issue_stage<C>(fill, rsrc_a, rsrc_b, rsrc_xs, rsrc_ws, lane_off_a, lane_off_b, q_stride, q_stride_b,
                               xs_off, fill_kb, wave, lane, C::fill_lo_j(j), C::fill_lo_j(j + 1), false);
            if (!C::kBlk32 && j > 0) {
#pragma unroll
                for (int i = 0; i < C::kTi; ++i)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        acc[i][j - 1][e] = __builtin_fmaf(tmp[c ^ 1][i][e], wsc, acc[i][j - 1][e]);
            }
            if (j + 1 < C::kTj) {
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) bcur[jj] = bnext[jj];
            }
        }
        if constexpr (!C::kBlk32) {
#pragma unroll
            for (int i = 0; i < C::kTi; ++i)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    acc[i][C::kTj - 1][e] = __builtin_fmaf(tmp[(C::kTj - 1) & 1][i][e], wsc, acc[i][C::kTj - 1][e]);
        }
      } else if constexpr (C::kX16) {
        // W8A16: per 16x16 tile and block, four 16x16x32 MFMAs on weights
        // widened in registers to their exact 16-bit values (widen8).  MFMA jj
        // of lane (r, g) takes K positions 16(g + 4(jj/2)) + 8(jj%2) .. +7:
        // weight bytes from chunks g and g + 4 of the fp8 row, and the
        // 16-bit token chunks 2g, 2g+1, 2g+8, 2g+9 of the 256-byte row.
        const float wsc = reinterpret_cast<const float*>(stage + C::kOffWs)[wave];
        u32x4 bfr[C::kTj][4];
#pragma unroll
        for (int j = 0; j < C::kTj; ++j) {
            const int row = C::kWaveM * wm + 16 * j + r;
#pragma unroll
            for (int jj = 0; jj < 4; ++jj)
                bfr[j][jj] = *reinterpret_cast<const u32x4*>(
                    stage + C::kStageA + swz_b16(row, 2 * g + 8 * (jj >> 1) + (jj & 1)));
        }
        float e0 = 1.0f, e1 = 1.0f;
        if constexpr (C::kBlk32) band_scales(stage, e0, e1);
        f32x4 tmp[2][C::kTj];
        i32x8 af = read_frag<true>(stage, a_base + a_row(0, r), g);
#pragma unroll
        for (int i = 0; i < C::kTi; ++i) {
            const int c = i & 1;
            const u32x4 aop[4] = {widen8<C::kXBf16>((uint32_t)af[0], (uint32_t)af[1], e0),
                                  widen8<C::kXBf16>((uint32_t)af[2], (uint32_t)af[3], e0),
                                  widen8<C::kXBf16>((uint32_t)af[4], (uint32_t)af[5], e1),
                                  widen8<C::kXBf16>((uint32_t)af[6], (uint32_t)af[7], e1)};
            if (i + 1 < C::kTi) af = read_frag<true>(stage, a_base + a_row(i + 1, r), g);
#pragma unroll
            for (int j = 0; j < C::kTj; ++j) {
                if constexpr (C::kBlk32) {
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) acc[i][j] = mfma_f16_16x16x32(aop[jj], bfr[j][jj], acc[i][j]);
                } else {
                    f32x4 blk = zero;
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj)
                        blk = C::kXBf16 ? mfma_bf16_16x16x32(aop[jj], bfr[j][jj], blk)
                                        : mfma_f16_16x16x32(aop[jj], bfr[j][jj], blk);
                    tmp[c][j] = blk;
                }
            }
            if constexpr (decltype(refill)::value)
                issue_stage<C>(fill, rsrc_a, rsrc_b, rsrc_xs, rsrc_ws, lane_off_a, lane_off_b, q_stride, q_stride_b,
                               xs_off, fill_kb, wave, lane, C::fill_lo(i), C::fill_lo(i + 1), false);
            if (!C::kBlk32 && i > 0) {
#pragma unroll
                for (int j = 0; j < C::kTj; ++j)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        acc[i - 1][j][e] = __builtin_fmaf(tmp[c ^ 1][j][e], wsc, acc[i - 1][j][e]);
            }
        }
        if constexpr (!C::kBlk32) {
#pragma unroll
            for (int j = 0; j < C::kTj; ++j)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    acc[C::kTi - 1][j][e] = __builtin_fmaf(tmp[(C::kTi - 1) & 1][j][e], wsc, acc[C::kTi - 1][j][e]);
        }
      } else {
        const float wsc = reinterpret_cast<const float*>(stage + C::kOffWs)[wave];
        const float* xs_lds = reinterpret_cast<const float*>(stage + C::kOffXs);
        float sc[C::kTj];
#pragma unroll
        for (int j = 0; j < C::kTj; ++j) sc[j] = xs_lds[C::kWaveM * wm + 16 * j + r] * wsc;
        i32x8 bf[C::kTj];
#pragma unroll
        for (int j = 0; j < C::kTj; ++j) bf[j] = read_frag<false>(stage, b_row0 + 16 * j, g);
        f32x4 tmp[2][C::kTj];
        i32x8 af = read_frag<true>(stage, a_base + a_row(0, r), g);
#pragma unroll
        for (int i = 0; i < C::kTi; ++i) {
            const int c = i & 1;
#pragma unroll
            for (int j = 0; j < C::kTj; ++j) tmp[c][j] = mfma_e4m3_16x16x128(af, bf[j], zero);
            if constexpr (decltype(refill)::value)
                issue_stage<C>(fill, rsrc_a, rsrc_b, rsrc_xs, rsrc_ws, lane_off_a, lane_off_b, q_stride, q_stride_b,
                               xs_off, fill_kb, wave, lane, C::fill_lo(i), C::fill_lo(i + 1), false);
            if (i + 1 < C::kTi) af = read_frag<true>(stage, a_base + a_row(i + 1, r), g);
            if (i > 0) {
#pragma unroll
                for (int j = 0; j < C::kTj; ++j)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        acc[i - 1][j][e] = __builtin_fmaf(tmp[c ^ 1][j][e], sc[j], acc[i - 1][j][e]);
            }
        }
#pragma unroll
        for (int j = 0; j < C::kTj; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                acc[C::kTi - 1][j][e] = __builtin_fmaf(tmp[(C::kTi - 1) & 1][j][e], sc[j], acc[C::kTi - 1][j][e]);
      }
    };

    auto stage = [&](int64_t b) { return stages + (int)(b % C::kStages) * C::kStageStride; };
    // Prologue: the first S-1 blocks in flight.
#pragma unroll
    for (int p = 0; p + 1 < C::kStages; ++p)
        if (p < nkb)
            issue_stage<C>(stage(p), rsrc_a, rsrc_b, rsrc_xs, rsrc_ws, lane_off_a, lane_off_b, q_stride, q_stride_b, xs_off, kb0 + p, wave,
                           lane);
    // Steady state: blocks whose stage is refilled with block b + S - 1,
    // then the last S - 1 blocks with no refill (two loops, so the
    // accumulators never meet a branch between two copies of the MFMA code).
    // At the top of each block: this wave's loads of block b are done (those
    // of the younger blocks b+1 .. b+S-2 that exist may stay in flight), and
    // so are its LDS reads of block b-1.  After the barrier every wave's
    // block b is in LDS and no wave reads the stage of block b-1, which
    // receives block b+S-1.
    const int64_t steady = nkb - (C::kStages - 1) > 0 ? nkb - (C::kStages - 1) : 0;
    for (int64_t b = 0; b < steady; ++b) {
        wait_stage<C>(C::kStages - 2);
        stage_barrier();
        // The scale loads of the refill block first (two short
        // instructions), its tile loads between the MFMA rows.
        uint8_t* fill = stage(b + C::kStages - 1);
        issue_stage<C>(fill, rsrc_a, rsrc_b, rsrc_xs, rsrc_ws, lane_off_a, lane_off_b, q_stride, q_stride_b, xs_off,
                       kb0 + b + C::kStages - 1, wave, lane, 0, 0, true);
        compute(stage(b), std::true_type{}, fill, kb0 + b + C::kStages - 1);
    }
    for (int64_t b = steady; b < nkb; ++b) {
        const int64_t left = nkb - 1 - b;
        wait_stage<C>(left < C::kStages - 2 ? (int)left : C::kStages - 2);
        stage_barrier();
        compute(stage(b), std::false_type{}, nullptr, 0);
    }

    // By a_row(), the lane holds, for token m = m0 + kWaveM wm + 16 j + r,
    // outputs n = n0 + kWaveN wn + 32 p + 8 g + t (t = 0..7) in acc[2p][j]
    // (t < 4) and acc[2p+1][j] (t >= 4).
    const int nl0 = C::kWaveN * wn + 8 * g, ml0 = C::kWaveM * wm + r;
    static_assert(C::kTi % 2 == 0, "tile pairs");
    auto store_tile = [&]() {
#pragma unroll
        for (int j = 0; j < C::kTj; ++j) {
            const int64_t m = m0 + ml0 + 16 * j;
            if (m >= M) continue;
#pragma unroll
            for (int p = 0; p < C::kTi / 2; ++p) {
                const int64_t n = n0 + nl0 + 32 * p;
                if (n < N) store8(y, y_dtype, m * N + n, acc[2 * p][j], acc[2 * p + 1][j]);
            }
        }
    };
    if (splits == 1) {
        store_tile();
        return;
    }

    if constexpr (C::kSplit) {
        // Split K.  Every workgroup of a tile has the same thread -> output
        // mapping, so a split's partial tile is kept in thread order: slot
        // (i, j) of thread x at ((split * kSlots + i * kTj + j) * kThreads +
        // x) * 16 bytes, one contiguous KB per wave and slot.  The slots are
        // written with 16-byte agent-coherent (sc1) stores, which write
        // through to memory every XCD sees; after they complete (vmcnt 0) and
        // the workgroup barrier, one thread counts the arrival on a
        // device-scope atomic.  The last workgroup reads every split with
        // 16-byte agent-coherent loads, four splits per round trip, and sums
        // them in split order.
        constexpr int kSlots = C::kTi * C::kTj;
        constexpr int kChunk = 4;
        constexpr int kSc1 = 16;                      // cache-policy bit: device-coherent access
        float* tile_parts = partials + t * splits * (C::BN * C::BM);
        const __amdgpu_buffer_rsrc_t prs = __builtin_amdgcn_make_buffer_rsrc(
            tile_parts, 0, (int)(splits * C::BN * C::BM * 4), 0x00020000);
        auto slot_off = [&](int64_t s, int slot) {
            return (int)(((s * kSlots + slot) * C::kThreads + threadIdx.x) * 16);
        };
#pragma unroll
        for (int i = 0; i < C::kTi; ++i)
#pragma unroll
            for (int j = 0; j < C::kTj; ++j)
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, acc[i][j]), prs,
                                                       slot_off(split, i * C::kTj + j), 0, kSc1);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (threadIdx.x == 0)
            arrived = __hip_atomic_fetch_add(&counters[t], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __syncthreads();
        if (arrived != (uint32_t)(splits - 1)) return;

        // This workgroup's own part is still in registers (the same bits it
        // wrote): only the other splits are read back.
        f32x4 own[C::kTi][C::kTj];
#pragma unroll
        for (int i = 0; i < C::kTi; ++i)
#pragma unroll
            for (int j = 0; j < C::kTj; ++j) {
                own[i][j] = acc[i][j];
                acc[i][j] = zero;
            }
        // kGroup slots at a time (at most 8 x kChunk loads in flight: the
        // partials of a whole large tile would not fit in registers), each
        // summed over the splits in split order.
        constexpr int kGroup = kSlots < 8 ? kSlots : 8;
        static_assert(kSlots % kGroup == 0, "slot groups");
#pragma unroll
        for (int g0 = 0; g0 < kSlots; g0 += kGroup) {
            for (int64_t s0 = 0; s0 < splits; s0 += kChunk) {
                i32x4 v[kChunk][kGroup];
#pragma unroll
                for (int u = 0; u < kChunk; ++u) {
                    if (s0 + u >= splits || s0 + u == split) continue;
#pragma unroll
                    for (int q = 0; q < kGroup; ++q)
                        v[u][q] = __builtin_amdgcn_raw_buffer_load_b128(prs, slot_off(s0 + u, g0 + q), 0, kSc1);
                }
#pragma unroll
                for (int u = 0; u < kChunk; ++u) {
                    if (s0 + u >= splits) continue;
#pragma unroll
                    for (int q = 0; q < kGroup; ++q) {
                        const int i = (g0 + q) / C::kTj, j = (g0 + q) % C::kTj;
                        acc[i][j] += s0 + u == split ? own[i][j] : __builtin_bit_cast(f32x4, v[u][q]);
                    }
                }
            }
        }
        store_tile();
        if (threadIdx.x == 0) __hip_atomic_store(&counters[t], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

namespace {

enum class TileShape { k256, k256x128, k128, k64x128, k128x64, k16_256, k16_128, k16_64 };

struct TilePlan {
    TileShape shape;
    int64_t bn, bm, tiles_n, tiles_m, splits, kb_per_split;
};

TilePlan make_plan(TileShape s, int64_t bn, int64_t bm, int64_t M, int64_t N, int64_t K) {
    TilePlan p{s, bn, bm, (N + bn - 1) / bn, (M + bm - 1) / bm, 1, 0};
    const int64_t KB = K / 128;
    int64_t splits = 1;
    if (s == TileShape::k16_128 || s == TileShape::k16_64) {
        // About one workgroup per CU, each with at least 4 K blocks.
        while (p.tiles_n * p.tiles_m * splits < kCUs && KB / (splits * 2) >= 4) splits *= 2;
    }
    p.kb_per_split = (KB + splits - 1) / splits;
    p.splits = (KB + p.kb_per_split - 1) / p.kb_per_split;
    return p;
}

// W8A8 tile plan by estimated time ([ADA] "One tile doesn't fit all M"):
// among every shape and K split (1, 2, 4, 8 or 16, at least four 128-K
// blocks per split), the least of
//   rounds x blocks per split x t_block(shape) + (split ? t_split : 0),
// rounds = ceil(workgroups / 256 CUs).  t_block is the measured time of one
// 128-K block of one workgroup at the sustained clock (us; it is nearly the
// same whatever the tile, most of it fixed cost per block, so larger tiles
// pay it for more outputs): 256x256 2.03, 256x128 1.46, 128x128 0.90,
// 64x128 and 128x64 0.77 (a four-wave 128x128 variant with 64 x 64 wave
// tiles measured the same as the eight-wave one, within 5%).  t_split
// is the hand-off of the partial tiles (written through to memory, summed
// by the last workgroup of a tile): 3.4 us + 0.021 us per KB of the
// splits' partial tiles (splits x the tile in fp32), fitted to measured
// split plans (64 KB: 4.7-5.1 us, 128 KB: 6.1-6.6 us, 512 KB: 14 us) when
// the last workgroup still read its own part back; it now keeps that part
// in registers (4096 x 4096 M = 512, split 2: 22.0 -> 21.2 us).  Split
// plans are kept to one round of workgroups and 16 MiB of partial tiles.
// Measured against the rules this replaces (us, N x K, M): 4096 x 4096
// M = 512 24.6 -> 21.3 (128x128 split 2), M = 256 17.4 -> 16.3 (128x64
// split 2); 12288 x 4096 M = 64 23.9 -> 17.4 (128x64 split 2, 192
// workgroups instead of 384), M = 128 33.4 -> 22.5 (128x128 split 2).
namespace {
struct ShapeCost {
    TileShape shape;
    int bn, bm;
    bool split_ok;
    double block_us;
};
constexpr ShapeCost kW8A8Shapes[] = {
    {TileShape::k256, 256, 256, false, 2.03},   {TileShape::k256x128, 256, 128, false, 1.46},
    {TileShape::k128, 128, 128, true, 0.90},
    {TileShape::k64x128, 64, 128, true, 0.77},  {TileShape::k128x64, 128, 64, true, 0.77},
};
constexpr int64_t kMaxPartialBytes = (int64_t)16 << 20;

TilePlan split_plan(const ShapeCost& c, int64_t M, int64_t N, int64_t K, int64_t splits) {
    TilePlan p{c.shape, c.bn, c.bm, (N + c.bn - 1) / c.bn, (M + c.bm - 1) / c.bm, 1, 0};
    const int64_t KB = K / 128;
    p.kb_per_split = (KB + splits - 1) / splits;
    p.splits = (KB + p.kb_per_split - 1) / p.kb_per_split;
    return p;
}
}  // namespace

TilePlan plan_tile(int64_t M, int64_t N, int64_t K) {
    const int64_t KB = K / 128;
    TilePlan best{};
    double best_cost = -1.0;
    for (const ShapeCost& c : kW8A8Shapes) {
        for (int64_t splits = 1; splits <= 16; splits *= 2) {
            if (splits > 1 && (!c.split_ok || (KB + splits - 1) / splits < 4)) break;
            const TilePlan p = split_plan(c, M, N, K, splits);
            if (splits > 1 && p.splits != splits) break;
            const int64_t wgs = p.tiles_n * p.tiles_m * p.splits;
            const int64_t tile_bytes = (int64_t)c.bn * c.bm * 4;
            if (p.splits > 1 && (wgs > kCUs || wgs * tile_bytes > kMaxPartialBytes)) continue;
            double cost = (double)((wgs + kCUs - 1) / kCUs) * (double)p.kb_per_split * c.block_us;
            if (p.splits > 1) cost += 3.4 + 0.021 * (double)(p.splits * tile_bytes) / 1024.0;
            if (best_cost < 0.0 || cost < best_cost) {
                best = p;
                best_cost = cost;
            }
        }
    }
    return best;
}

// W8A16 (16-bit activations, M > 16): 128 weight rows x 128 tokens (64
// tokens for M <= 64), K split when that leaves the CUs short of
// workgroups.
TilePlan plan_tile16(int64_t M, int64_t N, int64_t K) {
    const TilePlan big = make_plan(TileShape::k16_256, 256, 128, M, N, K);
    if (big.tiles_n * big.tiles_m >= kCUs) return big;
    if (M <= 64) return make_plan(TileShape::k16_64, 128, 64, M, N, K);
    return make_plan(TileShape::k16_128, 128, 128, M, N, K);
}

size_t counter_bytes(const TilePlan& p) {
    return ((size_t)(p.tiles_n * p.tiles_m) * sizeof(uint32_t) + 255) / 256 * 256;
}

template <class C>
void launch(const TilePlan& p, const void* xq, const float* xs, const uint8_t* wq, const void* ws, void* y,
            int y_dtype, int64_t M, int64_t N, int64_t K, float* partials, uint32_t* counters,
            hipStream_t stream) {
    const dim3 grid((unsigned)(p.tiles_n * p.tiles_m * p.splits));
    hipLaunchKernelGGL(w8a8_tile_kernel<C>, grid, dim3(C::kThreads), 0, stream, xq, xs, wq, ws, y, y_dtype, M, N,
                       K, p.tiles_n, p.tiles_m, p.splits, p.kb_per_split, partials, counters);
}

}  // namespace

static size_t plan_workspace_bytes(const TilePlan& p) {
    if (p.splits == 1) return 0;
    return counter_bytes(p) + (size_t)(p.tiles_n * p.tiles_m * p.splits * p.bn * p.bm) * sizeof(float);
}

size_t tile_workspace_bytes(int64_t M, int64_t N, int64_t K) { return plan_workspace_bytes(plan_tile(M, N, K)); }

static int waves_of(TileShape s) {
    switch (s) {
        case TileShape::k256: return Cfg256::kWaves;
        case TileShape::k256x128: return Cfg256x128::kWaves;
        case TileShape::k128: return Cfg128::kWaves;
        case TileShape::k64x128: return Cfg64x128::kWaves;
        case TileShape::k128x64: return Cfg128x64::kWaves;
        case TileShape::k16_256: return Cfg16_256<kTileBf16>::kWaves;
        case TileShape::k16_128: return Cfg16_128<kTileBf16>::kWaves;
        default: return Cfg16_64<kTileBf16>::kWaves;
    }
}

static TileInfo info_of(const TilePlan& p) {
    return TileInfo{(int)p.bn, (int)p.bm, waves_of(p.shape), p.tiles_n * p.tiles_m, p.splits};
}

TileInfo tile_info(int64_t M, int64_t N, int64_t K) { return info_of(plan_tile(M, N, K)); }
TileInfo tile16_info(int64_t M, int64_t N, int64_t K) { return info_of(plan_tile16(M, N, K)); }

size_t tile16_workspace_bytes(int64_t M, int64_t N, int64_t K) { return plan_workspace_bytes(plan_tile16(M, N, K)); }

size_t tile_counter_bytes(int64_t M, int64_t N, int64_t K) {
    const TilePlan p = plan_tile(M, N, K);
    return p.splits > 1 ? counter_bytes(p) : 0;
}

// Counters and partial tiles of a split plan inside the workspace; false
// (launch nothing) when the plan splits K and no workspace was given.
static bool split_parts(const TilePlan& p, void* workspace, uint32_t*& counters, float*& partials) {
    counters = nullptr;
    partials = nullptr;
    if (p.splits > 1) {
        if (!workspace) return false;
        counters = static_cast<uint32_t*>(workspace);
        partials = reinterpret_cast<float*>(static_cast<char*>(workspace) + counter_bytes(p));
    }
    return true;
}

hipError_t launch_w8a16_tile(const void* x, bool x_bf16, const uint8_t* wq, const float* ws, void* y,
                             int y_dtype, int64_t M, int64_t N, int64_t K, void* workspace, hipStream_t stream) {
    const TilePlan p = plan_tile16(M, N, K);
    uint32_t* counters;
    float* partials;
    if (!split_parts(p, workspace, counters, partials)) return hipErrorInvalidValue;
    if (p.shape == TileShape::k16_256) {
        if (x_bf16) launch<Cfg16_256<kTileBf16>>(p, x, nullptr, wq, ws, y, y_dtype, M, N, K, partials, counters, stream);
        else launch<Cfg16_256<kTileF16>>(p, x, nullptr, wq, ws, y, y_dtype, M, N, K, partials, counters, stream);
    } else if (p.shape == TileShape::k16_64) {
        if (x_bf16) launch<Cfg16_64<kTileBf16>>(p, x, nullptr, wq, ws, y, y_dtype, M, N, K, partials, counters, stream);
        else launch<Cfg16_64<kTileF16>>(p, x, nullptr, wq, ws, y, y_dtype, M, N, K, partials, counters, stream);
    } else {
        if (x_bf16) launch<Cfg16_128<kTileBf16>>(p, x, nullptr, wq, ws, y, y_dtype, M, N, K, partials, counters, stream);
        else launch<Cfg16_128<kTileF16>>(p, x, nullptr, wq, ws, y, y_dtype, M, N, K, partials, counters, stream);
    }
    return hipGetLastError();
}

hipError_t launch_w8a16_blk32_tile(const void* x, const uint8_t* wq, const uint8_t* e8m0, void* y, int y_dtype,
                                   int64_t M, int64_t N, int64_t K, void* workspace, hipStream_t stream) {
    const TilePlan p = plan_tile16(M, N, K);
    uint32_t* counters;
    float* partials;
    if (!split_parts(p, workspace, counters, partials)) return hipErrorInvalidValue;
    if (p.shape == TileShape::k16_256)
        launch<Cfg16_256<kTileF16Blk32>>(p, x, nullptr, wq, e8m0, y, y_dtype, M, N, K, partials, counters, stream);
    else if (p.shape == TileShape::k16_64)
        launch<Cfg16_64<kTileF16Blk32>>(p, x, nullptr, wq, e8m0, y, y_dtype, M, N, K, partials, counters, stream);
    else
        launch<Cfg16_128<kTileF16Blk32>>(p, x, nullptr, wq, e8m0, y, y_dtype, M, N, K, partials, counters, stream);
    return hipGetLastError();
}

hipError_t launch_w8a8_tile(const uint8_t* xq, const float* xs, const uint8_t* wq, const float* ws,
                            void* y, int y_dtype, int64_t M, int64_t N, int64_t K, void* workspace,
                            hipStream_t stream) {
    const TilePlan p = plan_tile(M, N, K);
    uint32_t* counters;
    float* partials;
    if (!split_parts(p, workspace, counters, partials)) return hipErrorInvalidValue;
    switch (p.shape) {
        case TileShape::k256:
            launch<Cfg256>(p, xq, xs, wq, ws, y, y_dtype, M, N, K, partials, counters, stream);
            break;
        case TileShape::k256x128:
            launch<Cfg256x128>(p, xq, xs, wq, ws, y, y_dtype, M, N, K, partials, counters, stream);
            break;
        case TileShape::k128:
            launch<Cfg128>(p, xq, xs, wq, ws, y, y_dtype, M, N, K, partials, counters, stream);
            break;
        case TileShape::k64x128:
            launch<Cfg64x128>(p, xq, xs, wq, ws, y, y_dtype, M, N, K, partials, counters, stream);
            break;
        case TileShape::k128x64:
            launch<Cfg128x64>(p, xq, xs, wq, ws, y, y_dtype, M, N, K, partials, counters, stream);
            break;
        default:
            break;
    }
    return hipGetLastError();
}

}  // namespace bfp8
