// W8A8 blockwise GEMM, tiled kernel for M > 16 (prefill) on gfx950.
//
// Workgroup tile: 256 weight rows (n) x 256 tokens (m), K staged one
// 128-wide scale block at a time ([ARC] "What this adds": the K tile is the
// scale block, so each stage has one scale per row block and token).  Eight
// waves, two per SIMD, each owning 128 n x 64 m = 8 x 4 MFMA tiles of 16x16;
// two waves per SIMD let one wave's promotion FMAs run in the shadow of the
// other wave's MFMAs.  Each wave's fp32 accumulators, operand fragments
// and block temporaries fit its 256 registers without spilling ([ADA] "Where
// the registers went").
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
// global 16 bytes belong there), two LDS stages of 65 KB, so block kb+1 is in
// flight while block kb is multiplied; one barrier per block.  LDS rows are
// 128 bytes (eight 16-byte chunks); chunk c of row r is stored at chunk
// position c ^ (r & 7), which makes the MFMA fragment reads (16 rows, same
// chunk) conflict-free.  Fragment K order: MFMA K slot g (lanes 16g..16g+15)
// takes chunks g and g + 4 of the row, the same for both operands, so the
// contraction is over the same 128 K values.

#include "bfp8_device.hpp"
#include "bfp8_launch.hpp"

namespace bfp8 {

namespace {

constexpr int kBN = 256;                  // weight rows per workgroup
constexpr int kBM = 256;                  // tokens per workgroup
constexpr int kWavesN = 2, kWavesM = 4;   // eight waves, two per SIMD
constexpr int kWaves = kWavesN * kWavesM;
constexpr int kThreads = kWaves * kWave;
constexpr int kWaveN = kBN / kWavesN, kWaveM = kBM / kWavesM;   // per-wave tile
constexpr int kTi = kWaveN / 16, kTj = kWaveM / 16;
constexpr int kRowBytes = 128;            // one 128-K block of one row
constexpr int kStageA = kBN * kRowBytes;
constexpr int kStageB = kBM * kRowBytes;
constexpr int kRowsPerLoad = kWave * 16 / kRowBytes;                        // 8 rows per load instruction
constexpr int kLoadsPerWave = (kBN + kBM) / (kRowsPerLoad * kWaves);        // tile loads per wave per stage
constexpr int kLoadsA = kBN / (kRowsPerLoad * kWaves);                      // of which weight rows
constexpr int kXsLanes = kBM / kWaves;    // token scales loaded per wave
constexpr int kStageXs = kBM * 4;         // token scales of the block, fp32
constexpr int kStageWs = kWaves * 4;      // one weight scale per wave, fp32
constexpr int kOffXs = kStageA + kStageB;
constexpr int kOffWs = kOffXs + kStageXs;
constexpr int kStageBytes = kOffWs + kStageWs;
constexpr int kStageStride = (kStageBytes + 1023) / 1024 * 1024;
// Two LDS stages: while block kb is multiplied out of one, block kb+1 lands
// in the other.
constexpr int kStages = 2;
// Vector-memory operations one stage adds per wave: tile loads, the token
// scales and the weight scale.
constexpr int kVmemPerStage = kLoadsPerWave + 2;
static_assert(kStages * kStageStride <= 160 * 1024, "LDS budget");
static_assert((kBN + kBM) % (kRowsPerLoad * kWaves) == 0 && kBN % (kRowsPerLoad * kWaves) == 0, "load split");
static_assert(kXsLanes <= kWave && kWaveN % 128 == 0 || 128 % kWaveN == 0, "one weight-scale row per wave");

typedef __attribute__((address_space(3))) void lds_void;

// Byte offset in a stage of (row, 16-byte chunk c) after the XOR swizzle.
__device__ __forceinline__ int swz(int row, int c) { return row * kRowBytes + ((c ^ (row & 7)) << 4); }

// Issue this wave's direct-to-LDS loads of K block kb into a stage.
// Instruction q of wave w fills LDS rows 8*(W q + w) .. +7 of the stage (W =
// waves; weight rows first, then token rows); lane l fills granule l of those
// 1 KB, i.e. row 8*(W q + w) + l/8 at chunk position l%8, so it fetches
// logical chunk (l%8) ^ (l/8) of that row.  The lane's byte offset inside the
// tile is the same for every q up to q * 8W rows, which goes into the scalar
// offset together with the K block.  Rows past the end of the matrix lie
// outside the buffer descriptor's range and load as zeros.
// A raw buffer descriptor (gfx9: dword 3 = 0x00020000, untyped 32-bit
// data; offsets at or past num_records read as zero), kept in SGPRs.
typedef int i32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ i32x4 buffer_rsrc(const void* base, uint32_t num_records) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    i32x4 r = {(int)(uint32_t)a, (int)((uint32_t)(a >> 32) & 0xFFFFu), (int)num_records, 0x00020000};
    r[0] = __builtin_amdgcn_readfirstlane(r[0]);
    r[1] = __builtin_amdgcn_readfirstlane(r[1]);
    r[2] = __builtin_amdgcn_readfirstlane(r[2]);
    return r;
}

__device__ __forceinline__ uint32_t lds_address(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// Direct-to-LDS buffer loads, issued as inline assembly: the data goes to LDS
// at M0 + 16 * lane (4 * lane for the dword form) and is waited for with
// explicit vmcnt waits.  Written as asm so that the compiler's own wait
// insertion, which cannot tell the two LDS stages apart, does not drain the
// prefetch before every LDS read.
__device__ __forceinline__ void dma16(uint32_t lds, i32x4 rsrc, int voff, int soff) {
    asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, %3 offen lds"
                 :: "v"(voff), "s"(rsrc), "s"(lds), "s"(soff) : "memory");
}
__device__ __forceinline__ void dma4(uint32_t lds, i32x4 rsrc, int voff, int soff) {
    asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dword %0, %1, %3 offen lds"
                 :: "v"(voff), "s"(rsrc), "s"(lds), "s"(soff) : "memory");
}

__device__ __forceinline__ void issue_stage(uint8_t* stage, i32x4 rsrc_a, i32x4 rsrc_b, i32x4 rsrc_xs,
                                            i32x4 rsrc_ws, int lane_off, int xs_off, int64_t K, int64_t kb,
                                            int wave, int lane) {
    const int k_off = (int)(kb * kRowBytes);
    const uint32_t base = lds_address(stage);
#pragma unroll
    for (int q = 0; q < kLoadsPerWave; ++q) {
        const uint32_t lds = __builtin_amdgcn_readfirstlane(base + kRowsPerLoad * (kWaves * q + wave) * kRowBytes);
        if (q < kLoadsA) {
            dma16(lds, rsrc_a, lane_off,
                  __builtin_amdgcn_readfirstlane(k_off + (int)(kRowsPerLoad * kWaves * q * K)));
        } else {
            dma16(lds, rsrc_b, lane_off,
                  __builtin_amdgcn_readfirstlane(k_off + (int)(kRowsPerLoad * kWaves * (q - kLoadsA) * K)));
        }
    }
    // Token scales xs[m0 + kXsLanes * w + l, kb], lanes l < kXsLanes only (the
    // dword form writes M0 + 4 * lane for every active lane).
    if (lane < kXsLanes)
        dma4(__builtin_amdgcn_readfirstlane(base + kOffXs + 4 * kXsLanes * wave), rsrc_xs, xs_off,
             __builtin_amdgcn_readfirstlane((int)(kb * 4)));
    // This wave's weight scale ws[nb, kb], lane 0 only.
    if (lane == 0)
        dma4(__builtin_amdgcn_readfirstlane(base + kOffWs + 4 * wave), rsrc_ws, 0,
             __builtin_amdgcn_readfirstlane((int)(kb * 4)));
}

// Workgroup barrier without the memory fence of __syncthreads(): that fence
// would wait for every outstanding direct-to-LDS load, including the
// prefetch of the next stage.  Visibility is handled by explicit counter
// waits instead (own stage loads complete before the barrier; own LDS reads
// complete before the barrier that frees a stage for reuse); the empty asm
// statements keep the compiler from moving memory accesses across it.
__device__ __forceinline__ void stage_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

__device__ __forceinline__ i32x8 read_frag(const uint8_t* stage, int row, int g) {
    const u32x4 lo = *reinterpret_cast<const u32x4*>(stage + swz(row, g));
    const u32x4 hi = *reinterpret_cast<const u32x4*>(stage + swz(row, g + 4));
    return __builtin_bit_cast(i32x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

__device__ __forceinline__ void tile_of_block(int64_t bid, int64_t tiles_n, int64_t tiles_m,
                                              int64_t& tn, int64_t& tm) {
    // Workgroups are dealt round-robin to the 8 XCDs.  Give each XCD a
    // contiguous run of tile indices, and walk tiles in groups of 8 token
    // tiles per weight tile, so the workgroups resident on one XCD share
    // weight and token rows in that XCD's L2.
    const int64_t total = tiles_n * tiles_m;
    int64_t t = bid;
    if (total % 8 == 0) t = (bid % 8) * (total / 8) + bid / 8;
    constexpr int64_t kGroup = 8;
    const int64_t per_group = kGroup * tiles_n;
    const int64_t group = t / per_group;
    const int64_t first_m = group * kGroup;
    const int64_t group_m = tiles_m - first_m < kGroup ? tiles_m - first_m : kGroup;
    const int64_t in_group = t - group * per_group;
    tm = first_m + in_group % group_m;
    tn = in_group / group_m;
}

}  // namespace

__global__ __launch_bounds__(kThreads, 1) void w8a8_tile_kernel(
    const uint8_t* __restrict__ xq, const float* __restrict__ xs,
    const uint8_t* __restrict__ wq, const float* __restrict__ ws,
    void* __restrict__ y, int y_dtype, int64_t M, int64_t N, int64_t K,
    int64_t tiles_n, int64_t tiles_m) {
    __shared__ __attribute__((aligned(1024))) uint8_t stages[kStages * kStageStride];

    int64_t tn, tm;
    tile_of_block(blockIdx.x, tiles_n, tiles_m, tn, tm);
    const int64_t n0 = tn * kBN, m0 = tm * kBM;
    const int64_t KB = K / 128, NB = (N + 127) / 128;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave), lane = threadIdx.x % kWave;
    const int wn = wave % kWavesN, wm = wave / kWavesN;
    const int r = lane & 15, g = lane >> 4;

    // Buffer descriptors over this workgroup's weight rows, token rows and
    // token-scale rows; rows past N or M lie outside them and load as zeros.
    const int64_t rows_a = N - n0 < kBN ? N - n0 : kBN;
    const int64_t rows_b = M - m0 < kBM ? M - m0 : kBM;
    const i32x4 rsrc_a = buffer_rsrc(wq + n0 * K, (uint32_t)(rows_a * K));
    const i32x4 rsrc_b = buffer_rsrc(xq + m0 * K, (uint32_t)(rows_b * K));
    const i32x4 rsrc_xs = buffer_rsrc(xs + m0 * KB, (uint32_t)(rows_b * KB * 4));
    const int lane_off = (int)((8 * wave + (lane >> 3)) * K) + ((((lane & 7) ^ ((lane >> 3) & 7))) << 4);
    const int xs_off = (int)((kXsLanes * wave + lane) * KB * 4);

    // Weight scales: one row of ws per wave (its 128 weight rows share it).
    int64_t nb = (n0 + kWaveN * wn) / 128;
    nb = nb < NB ? nb : NB - 1;
    const i32x4 rsrc_ws = buffer_rsrc(ws + nb * KB, (uint32_t)(KB * 4));

    f32x4 acc[kTi][kTj];
#pragma unroll
    for (int i = 0; i < kTi; ++i)
#pragma unroll
        for (int j = 0; j < kTj; ++j) acc[i][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    const f32x4 zero = {0.0f, 0.0f, 0.0f, 0.0f};

    const int a_row0 = kWaveN * wn + r;           // + 16 i
    const int b_row0 = kBN + kWaveM * wm + r;     // + 16 j

    // Per block, per wave: kTi rows of kTj MFMAs (one per 16x16 tile) into
    // block temporaries; the FMAs that promote row i are issued after row
    // i+1's MFMAs, so the matrix core and the VALU work on different rows.
    // The token fragments and the scales of the block are read first; the
    // weight fragments are streamed one row ahead.
    auto compute = [&](const uint8_t* stage) {
        const float wsc = reinterpret_cast<const float*>(stage + kOffWs)[wave];
        const float* xs_lds = reinterpret_cast<const float*>(stage + kOffXs);
        float sc[kTj];
#pragma unroll
        for (int j = 0; j < kTj; ++j) sc[j] = xs_lds[kWaveM * wm + 16 * j + r] * wsc;
        i32x8 bf[kTj];
#pragma unroll
        for (int j = 0; j < kTj; ++j) bf[j] = read_frag(stage, b_row0 + 16 * j, g);
        f32x4 tmp[2][kTj];
        i32x8 af = read_frag(stage, a_row0, g);
#pragma unroll
        for (int i = 0; i < kTi; ++i) {
            const int c = i & 1;
#pragma unroll
            for (int j = 0; j < kTj; ++j) tmp[c][j] = mfma_e4m3_16x16x128(af, bf[j], zero);
            if (i + 1 < kTi) af = read_frag(stage, a_row0 + 16 * (i + 1), g);
            if (i > 0) {
#pragma unroll
                for (int j = 0; j < kTj; ++j)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        acc[i - 1][j][e] = __builtin_fmaf(tmp[c ^ 1][j][e], sc[j], acc[i - 1][j][e]);
            }
        }
#pragma unroll
        for (int j = 0; j < kTj; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                acc[kTi - 1][j][e] = __builtin_fmaf(tmp[(kTi - 1) & 1][j][e], sc[j], acc[kTi - 1][j][e]);
    };

    auto stage = [&](int64_t kb) { return stages + (int)(kb % kStages) * kStageStride; };
    issue_stage(stage(0), rsrc_a, rsrc_b, rsrc_xs, rsrc_ws, lane_off, xs_off, K, 0, wave, lane);
    for (int64_t kb = 0; kb < KB; ++kb) {
        // This wave's loads of block kb and its LDS reads of block kb-1 are
        // done; after the barrier every wave's block kb is in LDS and nobody
        // reads block kb-1's stage, which then receives block kb+1.
        __builtin_amdgcn_s_waitcnt(0x7 << 4);                  // vmcnt(0), lgkmcnt(0)
        stage_barrier();
        if (kb + 1 < KB)
            issue_stage(stage(kb + 1), rsrc_a, rsrc_b, rsrc_xs, rsrc_ws, lane_off, xs_off, K, kb + 1, wave, lane);
        compute(stage(kb));
    }

    // Epilogue: lane holds n = n0 + 128 wn + 16 i + 4 g + e (e = 0..3) of token m.
#pragma unroll
    for (int j = 0; j < kTj; ++j) {
        const int64_t m = m0 + kWaveM * wm + 16 * j + r;
        if (m >= M) continue;
#pragma unroll
        for (int i = 0; i < kTi; ++i) {
            const int64_t n = n0 + kWaveN * wn + 16 * i + 4 * g;
            if (n >= N) continue;
            const f32x4 v = acc[i][j];
            if (y_dtype == 2) {
                *reinterpret_cast<f32x4*>(static_cast<float*>(y) + m * N + n) = v;
            } else {
                uint32_t h[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) h[e] = y_dtype == 0 ? float_to_bf16_bits(v[e]) : float_to_f16_bits(v[e]);
                *reinterpret_cast<uint2*>(static_cast<uint16_t*>(y) + m * N + n) =
                    make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
            }
        }
    }
}

hipError_t launch_w8a8_tile(const uint8_t* xq, const float* xs, const uint8_t* wq, const float* ws,
                            void* y, int y_dtype, int64_t M, int64_t N, int64_t K, hipStream_t stream) {
    const int64_t tiles_n = (N + kBN - 1) / kBN, tiles_m = (M + kBM - 1) / kBM;
    hipLaunchKernelGGL(w8a8_tile_kernel, dim3((unsigned)(tiles_n * tiles_m)), dim3(kThreads), 0, stream,
                       xq, xs, wq, ws, y, y_dtype, M, N, K, tiles_n, tiles_m);
    return hipGetLastError();
}

}  // namespace bfp8
