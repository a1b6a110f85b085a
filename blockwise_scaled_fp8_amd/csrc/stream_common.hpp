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

#include <type_traits>

#include "bfp8_device.hpp"
#include "bfp8_launch.hpp"

namespace bfp8 {

constexpr int kStreamWaves = 16;
static_assert(kStreamWaves == kStreamLaunchWaves, "plan and launch agree");
constexpr int kStreamThreads = kStreamWaves * kWave;
// Words of the cross-wave reduction scratch (stream_finish): one 16x16 fp32
// tile per wave and the split-K arrival word.
constexpr int kStreamRedWords = kStreamWaves * 256 + 1;
// Kernels with per-wave weight slabs overlay that scratch on the slabs (64
// KB, unused once every wave has multiplied its last block, which a barrier
// before stream_finish ensures): 16 KB less LDS per workgroup lets two
// workgroups share a CU when the token rows are small (measured 13.2 ->
// 11.0 us on a 12288 x 4096 projection at M = 1, whose 768 workgroups
// otherwise run in three rounds of one per CU).
__device__ __forceinline__ float* slab_scratch(uint8_t* slabs) { return reinterpret_cast<float*>(slabs); }

// Workspace layout of a split-K plan: one uint32 counter per output tile
// (padded to 256 bytes), then splits fp32 16x16 tiles per output tile.
inline size_t stream_counter_bytes(const StreamPlan& p) {
    return ((size_t)(p.n_tiles * p.m_tiles) * sizeof(uint32_t) + 255) / 256 * 256;
}
// Counters and partial tiles of a split plan inside the workspace; false
// (the caller launches nothing) when the plan splits K and no workspace was
// given.
inline bool stream_workspace_parts(const StreamPlan& p, void* ws, uint32_t*& counters, float*& partials) {
    counters = nullptr;
    partials = nullptr;
    if (p.splits == 1) return true;
    if (!ws) return false;
    counters = static_cast<uint32_t*>(ws);
    partials = reinterpret_cast<float*>(static_cast<char*>(ws) + stream_counter_bytes(p));
    return true;
}

// ------------------------------------------- one-token dot products ----
// Shared by the W8A8 and W8A16 kernels for M = 1 (K <= kGemvMaxK): eight
// waves per workgroup, lane l of a wave covering K offsets 1024 c + 16 l of
// each 1 KB chunk c of its weight rows.  The kernels are instantiated for
// kC = 4, 8, 12 or 16 chunks (gemv_chunks: the fewest covering K), and issue
// every load of all kC chunks before the first product.  The token is read
// from memory once per workgroup and shared through LDS (gemv_x_issue,
// gemv_x_store): with every wave reading all of it from L2, a 16-bit token
// of K = 4096 moved twice the weights' bytes through the caches (W8A16
// N = K = 4096: 5.25-5.35 us; the fused quantiser, which already shared its
// codes this way, ran 5.0 us over the same weights).
constexpr int kGemvWaves = 8;
constexpr int kGemvMaxChunks = 16;
constexpr int64_t kGemvMaxK = 1024 * kGemvMaxChunks;
static_assert(kGemvMaxK == kOneTokenMaxK, "routing and kernels agree");
inline int gemv_chunks(int64_t K) { return K <= 4096 ? 4 : K <= 8192 ? 8 : K <= 12288 ? 12 : 16; }

// The first kU * 8 KB of the token (descriptor rx; bytes past its range
// load as zeros) copied into LDS by the workgroup: thread t loads the 16
// bytes of unit t + 512 u (u < kU) in gemv_x_issue, before its weight
// loads, and stores them in gemv_x_store, after them; a barrier follows.
// Unit U sits at LDS unit U ^ ((U >> 4) & 1), so that a wave reading units
// 2 l and then 2 l + 1 (a 16-bit chunk: 32 bytes per lane) hits 16
// distinct bank groups per 16 lanes in each read.
constexpr int kGemvThreads = kGemvWaves * kWave;
// Cache policy of weight loads that no other workgroup of the call repeats
// (the one-token kernels; the streaming kernels with one token tile):
// non-temporal (nt) from 8 MiB of weights up.  A plain read of rotated
// copies measured (us, default / nt): 2 MiB 2.43-2.56 / 2.57-2.64, 4 MiB
// 2.51-2.52 / 2.71-2.78, 8 MiB 3.45 / 3.30-3.34, 16 MiB 4.61-4.62 /
// 4.48-4.49, 32 MiB 6.83-6.85 / 6.70-6.72; sc0 or sc1 alone changed
// nothing.  The token, which every workgroup reads, keeps the default.
constexpr int kLoadNt = 2;                           // the nt bit of a buffer load's cache policy
constexpr int64_t kNtMinWeightBytes = (int64_t)8 << 20;
__host__ __device__ inline bool weights_nt(int64_t N, int64_t K) { return N * K >= kNtMinWeightBytes; }
__device__ __forceinline__ int gemv_x_unit(int u) { return u ^ ((u >> 4) & 1); }
template <int kU>
__device__ __forceinline__ void gemv_x_issue(__amdgpu_buffer_rsrc_t rx, i32x4 (&v)[kU]) {
#pragma unroll
    for (int u = 0; u < kU; ++u)
        v[u] = __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                             rx, 16 * ((int)threadIdx.x + kGemvThreads * u), 0, 0));
}
template <int kU>
__device__ __forceinline__ void gemv_x_store(uint8_t* x_lds, const i32x4 (&v)[kU]) {
#pragma unroll
    for (int u = 0; u < kU; ++u)
        *reinterpret_cast<i32x4*>(x_lds + 16 * gemv_x_unit((int)threadIdx.x + kGemvThreads * u)) = v[u];
}
__device__ __forceinline__ i32x4 gemv_x_read(const uint8_t* x_lds, int unit) {
    return *reinterpret_cast<const i32x4*>(x_lds + 16 * gemv_x_unit(unit));
}

// The 16 E4M3 codes of v (K order) widened to 8 bf16 pairs (pair d: K
// offsets 2d, 2d + 1); exact for every finite code.
__device__ __forceinline__ void e4m3x16_to_bf16x2(i32x4 v, uint32_t (&p)[8]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        p[2 * i] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((uint32_t)v[i], 1.0f, false));
        p[2 * i + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((uint32_t)v[i], 1.0f, true));
    }
}

// One lane's 16 products of a chunk: xp[d] holds two 16-bit values (bf16
// or fp16, K offsets 2d and 2d + 1), w 16 E4M3 weights (byte b: K offset
// b), each widened exactly to the same 16-bit type and multiplied by
// `scale` (a power of two).  Two v_dot2c chains over alternate pairs (two
// products per instruction, each exact in fp32, accumulated in fp32), then
// their sum.  All of a one-token kernel's loads land over the launch's last
// microseconds, so this arithmetic after the last load is exposed: 8
// conversions and 8 v_dot2c per lane and chunk, where widening both
// operands to fp32 and multiplying took 24 to 40 VALU operations.
template <bool kBf16>
__device__ __forceinline__ float lane_dot16(const uint32_t (&xp)[8], i32x4 w, float scale = 1.0f) {
    float d0 = 0.0f, d1 = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t q = (uint32_t)w[i];
        if constexpr (kBf16) {
            d0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, xp[2 * i]),
                                                 __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q, scale, false), d0, false);
            d1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, xp[2 * i + 1]),
                                                 __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q, scale, true), d1, false);
        } else {
            d0 = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, xp[2 * i]),
                                        __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(q, scale, false), d0, false);
            d1 = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, xp[2 * i + 1]),
                                        __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(q, scale, true), d1, false);
        }
    }
    return d0 + d1;
}

// v plus the value of the lane given by DPP control `ctl` (a lane move
// inside the ALU, no LDS round trip).
template <int ctl>
__device__ __forceinline__ float add_dpp(float v) {
    return v + __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), ctl, 0xF, 0xF, false));
}

// Sum of a lane's partial over the 8 lanes of its 128-K block (lanes 8 j ..
// 8 j + 7): every lane of the group returns the block's sum, in one fixed
// order.  The lane sums pair lanes i ^ 1, then i ^ 2 (quad permutes), then
// the other quad of the eight (half-row mirror: after the first two steps
// every lane of a quad holds the same value, so lane 7 - i stands for lane
// i ^ 4).
__device__ __forceinline__ float block_sum8(float d) {
    d = add_dpp<0xB1>(d);    // quad_perm [1, 0, 3, 2]: lane i ^ 1
    d = add_dpp<0x4E>(d);    // quad_perm [2, 3, 0, 1]: lane i ^ 2
    d = add_dpp<0x141>(d);   // row_half_mirror: the other quad
    return d;
}

// The values of lanes i and i ^ kD (kD = 16 or 32), lower lane first, in
// every lane i: v_permlane16_swap / v_permlane32_swap with both operands v
// exchange rows of 16 lanes (halves of the wave) inside the ALU, where
// __shfl_xor goes through an LDS permute (checked on the GPU over every
// lane).  Combining the pair with a commutative operation gives the same
// bits as combining v with __shfl_xor(v, kD).  The compiler's optimiser
// folds a sum of the two results into twice the first one (seen in its IR
// for lo + hi; the hardware returns different rows), so the second result
// goes through an empty register constraint it cannot see into before use.
template <int kD>
__device__ __forceinline__ void lane_pair(float v, float& lo, float& hi) {
    static_assert(kD == 16 || kD == 32, "row or half-wave exchange");
    const uint32_t u = __builtin_bit_cast(uint32_t, v);
    const auto p = kD == 16 ? __builtin_amdgcn_permlane16_swap(u, u, false, false)
                            : __builtin_amdgcn_permlane32_swap(u, u, false, false);
    uint32_t h = p[1];
    asm volatile("" : "+v"(h));
    lo = __builtin_bit_cast(float, (uint32_t)p[0]);
    hi = __builtin_bit_cast(float, h);
}
template <int kD>
__device__ __forceinline__ float add_pair(float v) {
    float lo, hi;
    lane_pair<kD>(v, lo, hi);
    return lo + hi;
}
template <int kD>
__device__ __forceinline__ float max_pair(float v) {
    float lo, hi;
    lane_pair<kD>(v, lo, hi);
    return fmaxf(lo, hi);
}

// Maximum over aligned groups of kLanes lanes (2 .. 64), all by lane moves
// inside the ALU (the half-row mirror and row rotation stand for i ^ 4 and
// i ^ 8 once the smaller groups agree, lane_pair for i ^ 16 and i ^ 32).
template <int kLanes>
__device__ __forceinline__ float group_max(float v) {
    auto max_dpp = [](float a, auto ctl) {
        return fmaxf(a, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, a), decltype(ctl)::value,
                                                                          0xF, 0xF, false)));
    };
    if constexpr (kLanes > 1) v = max_dpp(v, std::integral_constant<int, 0xB1>{});
    if constexpr (kLanes > 2) v = max_dpp(v, std::integral_constant<int, 0x4E>{});
    if constexpr (kLanes > 4) v = max_dpp(v, std::integral_constant<int, 0x141>{});
    if constexpr (kLanes > 8) v = max_dpp(v, std::integral_constant<int, 0x128>{});
    if constexpr (kLanes > 16) v = max_pair<16>(v);
    if constexpr (kLanes > 32) v = max_pair<32>(v);
    return v;
}

// Sum of the eight block groups' promoted sums of a lane (lanes 8 apart).
__device__ __forceinline__ float group_sum8(float v) {
    v = add_dpp<0x128>(v);   // row_ror 8: lane i ^ 8 within its row of 16
    v = add_pair<16>(v);     // lane i ^ 16
    v = add_pair<32>(v);     // lane i ^ 32
    return v;
}

// Sum over all 64 lanes in one fixed order (pairs, quads, eights by lane
// moves, then group_sum8); every lane returns the total.
__device__ __forceinline__ float wave_sum(float v) {
    v = add_dpp<0xB1>(v);
    v = add_dpp<0x4E>(v);
    v = add_dpp<0x141>(v);
    return group_sum8(v);
}

// ------------------------------------------------------ weight slabs ----
// The 16 weight rows of one 128-K block (2 KB), staged in LDS with two
// direct-to-LDS loads of whole 128-byte lines (8 rows each): a load
// instruction then covers 8 full cache lines instead of 16 half lines,
// which a read probe measured at 3.99 vs 4.64 us for 16 MiB.  Lane l of
// each load fetches row l/8 (+ 8), chunk (l%8) ^ (row & 7); the MFMA
// operand of lane (r, g) is then chunks g and g + 4 of row r, read back at
// positions c ^ (r & 7) (16 consecutive rows: conflict-free).
constexpr int kSlabBytes = 16 * 128;

// Lane offset of this lane's slab loads inside a 16-row window of W.
__device__ __forceinline__ int slab_lane_offset(int lane, int64_t K) {
    return (int)((lane >> 3) * K) + (((lane & 7) ^ ((lane >> 3) & 7)) << 4);
}

// Issue the two loads of block kb of the 16 rows that `rsrc` covers;
// non-temporal when `nt` (wave-uniform: no other workgroup of the call
// reads the same weights, and they are large enough, weights_nt).
__device__ __forceinline__ void slab_issue(uint8_t* slab, i32x4 rsrc, int lane_off, int64_t K, int64_t kb,
                                           bool nt) {
    const uint32_t lds = __builtin_amdgcn_readfirstlane(lds_address(slab));
    const int k_off = __builtin_amdgcn_readfirstlane((int)(kb * 128));
    const int row8 = __builtin_amdgcn_readfirstlane((int)(8 * K));
    if (nt) {
        dma16_nt(lds, rsrc, lane_off, 0, k_off);
        dma16_nt(lds + 1024, rsrc, lane_off, row8, k_off);
    } else {
        dma16(lds, rsrc, lane_off, 0, k_off);
        dma16(lds + 1024, rsrc, lane_off, row8, k_off);
    }
}

__device__ __forceinline__ void slab_read(const uint8_t* slab, int r, int g, u32x4& lo, u32x4& hi) {
    lo = *reinterpret_cast<const u32x4*>(slab + r * 128 + ((g ^ (r & 7)) << 4));
    hi = *reinterpret_cast<const u32x4*>(slab + r * 128 + (((g + 4) ^ (r & 7)) << 4));
}

// ------------------------------------------------------ token rows ----
// The token rows of one 128-K block staged in LDS by direct-to-LDS dword
// loads: 256 bytes (128 16-bit values) per token, rows padded to
// kXRowStride bytes so that the same column of consecutive rows falls in
// distinct banks.  The loads are issued before a block's weight slabs, so
// (loads complete in issue order) a wave can wait for its token rows while
// the weights are still in flight.
constexpr int kXRowStride = 272;   // 256-byte token rows, padded: rows of one column land in distinct banks

// Direct-to-LDS loads of the kMp token rows of block kb into `rows` (one
// dword per lane per row).  Rows at or past M lie past the descriptor's
// range and load as zeros.
template <int kMp>
__device__ __forceinline__ void xrows_issue(uint8_t* rows, i32x4 rsrc_x, int lane, int64_t K, int64_t kb) {
    const uint32_t base = __builtin_amdgcn_readfirstlane(lds_address(rows));
    const int k_off = __builtin_amdgcn_readfirstlane((int)(kb * 256));
#pragma unroll
    for (int t = 0; t < kMp; ++t)
        dma4(__builtin_amdgcn_readfirstlane(base + t * kXRowStride), rsrc_x, (int)(t * K * 2) + 4 * lane, k_off);
}

// s_waitcnt vmcnt(N) alone; also a compiler barrier for memory accesses.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N == 0 || N == 2 || N == 4, "wait counts used here");
    if constexpr (N == 0) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    else if constexpr (N == 2) asm volatile("s_waitcnt vmcnt(2)" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
}

// A pass of a streaming kernel issues its loads block by block (token rows
// of both blocks, then the weight slabs of block 0, then those of block 1).
// Loads complete in issue order, so block 0 is in once at most the two slab
// loads of block 1 are outstanding: the wave multiplies block 0 while block
// 1 is still arriving.  `two`: this pass has a block 1 (wave-uniform).
__device__ __forceinline__ void wait_block(int c, bool two) {
    if (c == 0 && two) wait_vmcnt<2>();
    else wait_vmcnt<0>();
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

// red: LDS scratch of kStreamRedWords words (the wave tiles, then the
// arrival word of the split-K hand-off).  Must be called by every thread of
// the workgroup (it contains barriers).
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
    uint32_t* arrived = reinterpret_cast<uint32_t*>(red + kStreamWaves * 256);
    if (t == 0) *arrived = __hip_atomic_fetch_add(&counters[tile], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    if (*arrived != (uint32_t)(splits - 1)) return;   // not the last workgroup of this tile

    if (t < 256) {
        // Sum in split order; the loads of eight splits are issued together
        // before any is added (one memory round trip per eight splits).  This
        // workgroup's own part is v, the same bits it wrote.
        constexpr int kChunk = 8;
        float s = 0.0f;
        for (int64_t k0 = 0; k0 < splits; k0 += kChunk) {
            float p[kChunk];
#pragma unroll
            for (int u = 0; u < kChunk; ++u)
                if (k0 + u < splits)
                    p[u] = k0 + u == split ? v
                                           : __hip_atomic_load(&my_tiles[(k0 + u) * 256 + t], __ATOMIC_RELAXED,
                                                               __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
            for (int u = 0; u < kChunk; ++u)
                if (k0 + u < splits) s += p[u];
        }
        if (m < M) store_out(y, y_dtype, m * N + n, s);
    }
    if (t == 0) __hip_atomic_store(&counters[tile], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);   // re-arm
}

}  // namespace bfp8
