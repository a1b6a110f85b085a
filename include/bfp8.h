/*
 * bfp8.h — C ABI of libbfp8, the blockwise-scaled FP8 GEMM library for
 * AMD Instinct MI355X (gfx950).
 *
 * Pages cited (by title and section):
 *   [ADA]  "Blockwise FP8 on Ada GPUs, part 2: my kernel was correct and 4x
 *          too slow"
 *   [ARC]  "perf(ArcKernels): blockwise-FP8 GEMM on tensor cores, scale
 *          promoted per 128-K" (including its "Route-2 handover" comment)
 *   [SM70] "SM70 FP8 block-32 kernels (PLI Labs)"
 *   [3090] "FP8 / NVFP4 の weight-only 推論で RTX 3090 が失っているものは無い"
 *
 * Conventions shared by every entry point
 *   - Matrices are row-major.  Weights are W[N, K] with K contiguous and every
 *     product is Y[M, N] = X[M, K] . W^T ("TN", [ARC] "Route-2 handover"
 *     item 4; [SM70] "Build and use", weights [N, K] and scales [N/32, K/32]).
 *   - E4M3 means the OCP "fn" 8-bit format: bias 7, subnormals, no infinity,
 *     0x7F / 0xFF are NaN, largest magnitude 448 ([ARC] "What this adds";
 *     [SM70] "Exactness").
 *   - Device pointers are caller-owned device memory; the library allocates
 *     nothing and keeps no state between calls.  Every device pointer must
 *     be 16-byte aligned.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Work is enqueued asynchronously on it; the library never synchronises.
 *   - Every argument is validated before any HIP call.  A failed check
 *     returns a nonzero bfp8_status and enqueues nothing.  No entry point
 *     aborts, throws or prints.  A HIP launch failure returns
 *     BFP8_E_LAUNCH.
 *   - Preconditions not checked on the hot path: inputs and scales finite,
 *     scales >= 0, no E4M3 NaN codes in device operands (the host-side
 *     bfp8_prepare_blk32_ue8m0 checks its operands), no overlap between
 *     outputs and inputs.
 *   - Determinism: every reduction is done in a fixed order (no
 *     floating-point atomics); two calls on the same inputs give the same bits.
 */
#ifndef BFP8_H
#define BFP8_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int bfp8_status;

enum {
    BFP8_OK = 0,
    BFP8_E_NULL = 1,            /* a required pointer is NULL */
    BFP8_E_SHAPE = 2,           /* a size is out of range or not a required multiple */
    BFP8_E_DTYPE = 3,           /* unknown or unsupported dtype code */
    BFP8_E_ALIGN = 4,           /* a device pointer is not 16-byte aligned */
    BFP8_E_WORKSPACE = 5,       /* workspace missing or smaller than bfp8_workspace_bytes() */
    BFP8_E_NAN_CODE = 6,        /* E4M3 NaN code (0x7F / 0xFF) in a weight */
    BFP8_E_SCALE_NOT_POW2 = 7,  /* block scale not a positive finite power of two */
    BFP8_E_SCALE_WINDOW = 8,    /* power-of-two scale 2^e with e outside [-14, 7] */
    BFP8_E_LAUNCH = 9,          /* the HIP runtime refused a launch */
    BFP8_E_OP = 10              /* unknown op code */
};

/* dtype codes of 16-bit/32-bit operands */
enum { BFP8_BF16 = 0, BFP8_F16 = 1, BFP8_F32 = 2 };

/* op codes for bfp8_workspace_bytes / bfp8_get_limits */
enum {
    BFP8_OP_QUANT_ACT_1X128 = 0,
    BFP8_OP_QUANT_WEIGHT_128X128 = 1,
    BFP8_OP_GEMM_W8A8_BLK128 = 2,
    BFP8_OP_GEMM_W8A16_BLK128 = 3,
    BFP8_OP_GEMM_W8A16_BLK32_UE8M0 = 4,
    BFP8_OP_QUANT_GEMM_W8A8_BLK128 = 5
};

/*
 * 1x128 activation quantisation ([ADA] "The starting point": one scale per
 * token per 128 values along K; [ARC] "Route-2 handover" item 2: scales of
 * shape [M, ceil(K/128)]; item 3: one wave per group with a register
 * reduction and vector loads instead of 1024-thread blocks and serialised
 * atomics).
 *   x   [M, K] bf16 or fp16 (x_dtype BFP8_BF16 / BFP8_F16), device.
 *   xq  [M, K] E4M3 codes, device, written.
 *   xs  [M, ceil(K/128)] fp32, row-major, device, written.
 * Per row m and group g (columns [128g, min(K, 128g+128))):
 *   amax = max |x|;  s = fl32(amax / 448);  q = RNE-saturating E4M3 of
 *   fl32(x / s) (IEEE fp32 divisions); amax == 0 gives s = 0 and codes 0x00.
 * The codes and scales are bit-exact functions of x.
 * Requires M >= 1, K >= 8, K % 8 == 0 (the last group may be ragged).
 */
bfp8_status bfp8_quantize_act_1x128(const void* x, int x_dtype, int64_t M, int64_t K,
                                    uint8_t* xq, float* xs, void* stream);

/*
 * 128x128 weight quantisation, the load-time preparation of W8A8/W8A16
 * blk128 weights ([ADA] "The starting point": 128x128 weight blocks;
 * [ARC] "What this adds": the [N/128, K/128] block scale).
 *   w   [N, K] bf16 or fp16, device.
 *   wq  [N, K] E4M3 codes, device, written.
 *   ws  [ceil(N/128), ceil(K/128)] fp32, row-major, device, written.
 * Per tile: the same amax / scale / code rule as the activation quantiser.
 * Requires N >= 1, K >= 8, K % 8 == 0 (edge tiles may be ragged).
 */
bfp8_status bfp8_quantize_weight_128x128(const void* w, int w_dtype, int64_t N, int64_t K,
                                         uint8_t* wq, float* ws, void* stream);

/*
 * Blockwise weight dequantisation at load time: the fallback for a layer
 * whose 32x32 scales bfp8_prepare_blk32_ue8m0 refuses ([SM70] "Exactness":
 * only power-of-two scales in [2^-14, 2^7] keep the block-32 weights exact in
 * fp16; other layers are dequantised once when loaded).  Per-step
 * dequantisation is what the pages warn against ([ARC] "Route-2 handover"),
 * so this is meant for load time: dequantise, then requantise the result with
 * bfp8_quantize_weight_128x128 and run the blk128 GEMMs on it.
 *   wq      [N, K] E4M3 codes, device.
 *   scales  [ceil(N/block), ceil(K/block)] fp32, row-major, device (any
 *           values; no window or power-of-two rule applies here).
 *   block   32 or 128.
 *   w       [N, K] in w_dtype (BFP8_BF16, BFP8_F16 or BFP8_F32), device, written.
 * w[n, k] = RN(fl32(E4M3(wq[n, k]) * scales[n / block, k / block])): the fp32
 * product rounded to nearest even to w_dtype (fp32 output is the product).
 * NaN codes (0x7F, 0xFF) give NaN.  Requires N >= 1, K >= 8, K % 8 == 0 (edge
 * blocks may be ragged); pointers 16-byte aligned.  Asynchronous on `stream`;
 * errors: BFP8_E_NULL, BFP8_E_SHAPE (including a block other than 32 or 128),
 * BFP8_E_DTYPE, BFP8_E_ALIGN, BFP8_E_LAUNCH.
 */
bfp8_status bfp8_dequantize_weight(const uint8_t* wq, const float* scales, int64_t block, void* w, int w_dtype,
                                   int64_t N, int64_t K, void* stream);

/*
 * W8A8 blockwise GEMM ([ADA] "The starting point" and "The fix"; [ARC]
 * "What this adds"):
 *   for each 128-wide K block kb:
 *     P[m, n]  = sum over k in kb of E4M3(xq[m, k]) * E4M3(wq[n, k])   (FP8 MFMA, fp32)
 *     Y[m, n] += P[m, n] * xs[m, kb] * ws[n / 128, kb]                 (once per block)
 *   xq  [M, K] E4M3, xs [M, K/128] fp32 (from bfp8_quantize_act_1x128).
 *   wq  [N, K] E4M3, ws [ceil(N/128), K/128] fp32.
 *   y   [M, N], y_dtype BFP8_BF16 / BFP8_F16 / BFP8_F32 (round to nearest even
 *       from the fp32 accumulator).
 *   workspace: device memory of at least bfp8_workspace_bytes(
 *       BFP8_OP_GEMM_W8A8_BLK128, M, N, K) bytes (may be NULL when that is 0).
 *       It must be zero-filled before its first use; every call leaves it
 *       ready for the next.  Calls that overlap in time must not share one.
 * Requires M >= 1, N >= 16, N % 16 == 0, K >= 128, K % 128 == 0, K <= 2^23.
 */
bfp8_status bfp8_gemm_w8a8_blk128(const uint8_t* xq, const float* xs,
                                  const uint8_t* wq, const float* ws,
                                  void* y, int y_dtype, int64_t M, int64_t N, int64_t K,
                                  void* workspace, size_t workspace_bytes, void* stream);

/*
 * The W8A8 blockwise GEMM for callers that cannot allocate: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  Same
 * arguments, kernels and results (bit for bit) as bfp8_gemm_w8a8_blk128,
 * without the workspace arguments: the library keeps one device array of
 * BFP8_NOALLOC_SCRATCH_BYTES per GPU (static device memory, held from the
 * library's first use on that GPU until the process ends) and uses it as
 * the workspace.  The call allocates nothing and calls no allocating
 * routine; on its first call on a GPU it looks up that GPU's copy of the
 * array (hipGetSymbolAddress, no allocation).  When the plan splits K it
 * first clears the plan's tile counters with a small kernel on `stream`
 * (no memset, so the call can be captured into a graph).
 * Every call on one GPU shares that GPU's array: calls that may overlap in
 * time on one GPU (other streams, other threads, graphs replayed
 * concurrently) race and must be serialised by the caller.
 * Shapes whose workspace (bfp8_workspace_bytes(BFP8_OP_GEMM_W8A8_BLK128,
 * M, N, K)) exceeds BFP8_NOALLOC_SCRATCH_BYTES return BFP8_E_WORKSPACE (the
 * planners keep every shape within it: at most 16 MiB + 512 bytes).
 * Other errors as for bfp8_gemm_w8a8_blk128; BFP8_E_LAUNCH also when the
 * array cannot be located on the current device.
 */
#define BFP8_NOALLOC_SCRATCH_BYTES ((size_t)(16u << 20) + 4096u)
bfp8_status bfp8_gemm_w8a8_blk128_noalloc(const uint8_t* xq, const float* xs,
                                          const uint8_t* wq, const float* ws,
                                          void* y, int y_dtype, int64_t M, int64_t N, int64_t K, void* stream);

/*
 * Activation quantisation fused with the W8A8 blockwise GEMM.  [ADA]
 * "Results on the L4" counts the activation quantisation inside the GEMM's
 * time and "What's not good yet" names batch-1 decode as the gap; fusing
 * removes a launch and the codes' round trip through memory at decode.
 * Computes exactly bfp8_quantize_act_1x128 followed by bfp8_gemm_w8a8_blk128
 * on the same arguments: the same codes, scales and per-block promotion, so
 * y is bit-identical to that pair of calls.
 *   x   [M, K] bf16 or fp16 (x_dtype BFP8_BF16 / BFP8_F16), device.
 *   wq, ws, y, y_dtype: as for bfp8_gemm_w8a8_blk128.
 *   workspace: at least bfp8_workspace_bytes(BFP8_OP_QUANT_GEMM_W8A8_BLK128,
 *       M, N, K) bytes, zero-filled before its first use, left ready for the
 *       next call; calls that overlap in time must not share one.  For M = 1
 *       with K <= 8192 (the one-token kernel; no workspace) and for M <= 8
 *       where bfp8_gemm_w8a8_blk128 uses the weight-streaming kernel, the
 *       kernel quantises the activations itself; otherwise the codes and
 *       scales are staged in the workspace by the 1x128 quantiser.
 * Requires M >= 1, N >= 16, N % 16 == 0, K >= 128, K % 128 == 0, K <= 2^23.
 */
bfp8_status bfp8_quant_gemm_w8a8_blk128(const void* x, int x_dtype,
                                        const uint8_t* wq, const float* ws,
                                        void* y, int y_dtype, int64_t M, int64_t N, int64_t K,
                                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * W8A16 blockwise GEMM: 16-bit activations, E4M3 weights widened to the
 * activations' type in registers by the FP8 conversion instructions
 * ([3090] §2, §4.1: the widening is exact; [ARC] "What this adds": the
 * scale is applied once per 128 K values).
 *   Y[m, n] = sum_kb ws[n / 128, kb] * sum over k in kb of x[m, k] * E4M3(wq[n, k])
 *   x   [M, K] bf16 or fp16, wq [N, K] E4M3, ws [ceil(N/128), K/128] fp32.
 *   y   [M, N] in y_dtype (BF16 / F16 / F32); workspace as for W8A8 (sized
 *       by bfp8_workspace_bytes(BFP8_OP_GEMM_W8A16_BLK128, M, N, K)).
 * M = 1 with K <= 12288 runs a dot-product kernel on the vector ALUs (two
 * 16-bit products per instruction); M <= 16 otherwise streams the weights
 * (decode);
 * larger M reads all tokens per weight tile or runs a tiled MFMA kernel that
 * widens each weight fragment once per wave and reuses it for up to 64
 * tokens ([3090] §4.4: at prefill the weight-only cost is a few percent).
 * Requires M >= 1, N % 16 == 0, K % 128 == 0, K <= 2^23.
 */
bfp8_status bfp8_gemm_w8a16_blk128(const void* x, int x_dtype,
                                   const uint8_t* wq, const float* ws,
                                   void* y, int y_dtype, int64_t M, int64_t N, int64_t K,
                                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * W8A16 GEMM with 32x32 weight tiles and power-of-two (UE8M0) scales
 * ([SM70] "How it works", "Exactness"): each weight is widened to fp16 and
 * multiplied by its tile's 2^e in one conversion instruction (exact in fp16
 * for e in [-14, 7]), then contracted with fp32 accumulation.  One token
 * with K <= 8192 runs a dot-product kernel on the vector ALUs, M <= 16
 * otherwise streams the weights, larger M streams them once per 16 tokens.
 *   Y[m, n] = sum_k x[m, k] * (E4M3(wq[n, k]) * 2^(e8m0[n/32, k/32] - 127))
 *   x     [M, K] fp16 (x_dtype BFP8_F16).
 *   wq    [N, K] E4M3.
 *   e8m0  [N/32, K/32] bytes E, produced by bfp8_prepare_blk32_ue8m0
 *         (trusted: E must lie in [113, 134]).
 *   y     [M, N] in y_dtype (F16 / BF16 / F32); workspace as for W8A8.
 * Requires M >= 1, N % 32 == 0, K % 128 == 0, K <= 2^23.
 */
bfp8_status bfp8_gemm_w8a16_blk32_ue8m0(const void* x, int x_dtype,
                                        const uint8_t* wq, const uint8_t* e8m0,
                                        void* y, int y_dtype, int64_t M, int64_t N, int64_t K,
                                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * Load-time validation and packing of 32x32 power-of-two scales ([SM70]
 * "Exactness": the packer refuses, loudly, scales outside [2^-14, 2^7],
 * scales that are not powers of two, and E4M3 NaN codes).  HOST memory,
 * synchronous, touches no GPU.
 *   wq_host     [N, K] E4M3 codes.
 *   scale_host  [N/32, K/32] fp32 scales.
 *   e8m0_host   [N/32, K/32] bytes, written only on success: E = e + 127.
 *   bad_index   written always: -1 on success, else the flat row-major index
 *               of the first offending element (weights are checked first,
 *               then scales).
 * Returns BFP8_E_NAN_CODE, BFP8_E_SCALE_NOT_POW2 (zero, negative, infinite,
 * NaN or non-power-of-two scale) or BFP8_E_SCALE_WINDOW (2^e, e outside
 * [-14, 7]) on refusal.  Requires N >= 32 with N % 32 == 0, and K >= 128
 * with K % 128 == 0: the 32x32 tiles of the format, in whole 128-K blocks,
 * the unit bfp8_gemm_w8a16_blk32_ue8m0 streams, so that every layer this
 * packer accepts is one that GEMM accepts (BFP8_E_SHAPE otherwise).
 */
bfp8_status bfp8_prepare_blk32_ue8m0(const uint8_t* wq_host, const float* scale_host,
                                     int64_t N, int64_t K, uint8_t* e8m0_host,
                                     int64_t* bad_index);

/* Bytes of workspace the op needs for this shape (0 when none). */
size_t bfp8_workspace_bytes(int op, int64_t M, int64_t N, int64_t K);

/*
 * Shape rules compiled into the kernels, read from the library rather than
 * duplicated by callers ([ARC] "Correctness guards": eligibility read from
 * the kernel so host checks cannot drift from the compiled tiling).
 *   k_multiple    K must be a multiple of this.
 *   n_multiple    N must be a multiple of this.
 *   align_bytes   required alignment of every device pointer.
 *   m_stream_max  largest M served by the small-M (decode) kernels, one
 *                 16-token MFMA tile.  One token runs a dot-product kernel
 *                 on the vector ALUs: with K <= 8192 for W8A8, the fused
 *                 call and blk32, K <= 12288 for W8A16.  Otherwise W8A8
 *                 streams the weights when K needs no split across
 *                 workgroups, or N < 1024, except that above 4 tokens
 *                 (with K <= 4096) where streaming would take several
 *                 rounds of workgroups, and above m_stream_max / 2 tokens
 *                 where it would leave CUs idle, a kernel that reads all
 *                 tokens of a 16-token tile per 16-, 32- or 64-row weight
 *                 tile runs instead; up to 4 * m_stream_max it also streams
 *                 one workgroup per 16-token tile when those workgroups
 *                 fit one round on the CUs without a split of K.  The
 *                 all-token kernel serves the other M <= 2 * m_stream_max
 *                 (splitting K over two or four workgroups at K >= 12288
 *                 where one workgroup per weight tile would leave most CUs
 *                 idle, and over two for 32-row tiles in place of 16-row
 *                 ones above m_stream_max tokens, which halves the token
 *                 rows each workgroup reads), and K <= 4096 where M * N <= 2^19 or, for
 *                 N >= 512, its launch fits one round of workgroups on the
 *                 CUs; the tiled MFMA kernels otherwise.  W8A16 blk128 and
 *                 blk32 stream M <= m_stream_max / 2 (W8A16 blk128 at
 *                 M >= 4 with K <= 4096 runs the all-token kernel where
 *                 streaming would take several rounds); for m_stream_max /
 *                 2 < M <= m_stream_max they run the all-token kernel with
 *                 one 16-token tile unless the streaming plan would split
 *                 K (then they stream).  Above m_stream_max, W8A16 blk128
 *                 reads all tokens per weight tile when K <= 4096 and
 *                 either M <= 2 * m_stream_max or that launch fits one
 *                 round of workgroups, and for M <= 4 * m_stream_max when
 *                 K <= 8192 and the launch fits one round, and uses its
 *                 tiled MFMA kernel otherwise; blk32 reads all tokens for
 *                 M <= 16 * m_stream_max when K <= 4096 and either M <= 2 *
 *                 m_stream_max or M * N <= 2^19, and for M <= 2 *
 *                 m_stream_max when K <= 8192 in one round (its tiled form,
 *                 scales applied in the widening, has no promotion step),
 *                 and streams one 16-token tile per workgroup where that
 *                 plan splits K.
 * Any output pointer may be NULL.
 */
bfp8_status bfp8_get_limits(int op, int64_t* k_multiple, int64_t* n_multiple,
                            int64_t* align_bytes, int64_t* m_stream_max);

/*
 * Kernels a call can run, as reported by bfp8_get_plan.  One tile does not
 * fit every M ([ADA] "One tile doesn't fit all M"; [SM70] "How it works":
 * GEMV-style kernels for a few tokens, matrix-core tiles above), so each
 * GEMM picks one of these by M, N and K.
 */
enum {
    BFP8_KERNEL_NONE = 0,
    BFP8_KERNEL_QUANT_ACT = 1,          /* 1x128 activation quantiser */
    BFP8_KERNEL_QUANT_WEIGHT = 2,       /* 128x128 weight quantiser */
    BFP8_KERNEL_W8A8_GEMV = 3,          /* one token, codes in: dot products on the vector ALUs */
    BFP8_KERNEL_W8A8_GEMV_QUANT = 4,    /* one token, 16-bit in, quantised inside the kernel */
    BFP8_KERNEL_W8A8_STREAM = 5,        /* weight-streaming MFMA kernel, 16-token tiles, codes in */
    BFP8_KERNEL_W8A8_STREAM_QUANT = 6,  /* weight-streaming MFMA kernel, quantised inside the kernel */
    BFP8_KERNEL_W8A8_WIDE = 7,          /* all tokens of a group per 16/32-row weight tile */
    BFP8_KERNEL_W8A8_TILE = 8,          /* tiled MFMA kernel */
    BFP8_KERNEL_W8A16_GEMV = 9,         /* one token: dot products on the vector ALUs */
    BFP8_KERNEL_W8A16_STREAM = 10,      /* weight-streaming MFMA kernel */
    BFP8_KERNEL_W8A16_WIDE = 11,        /* all tokens of a group per weight tile */
    BFP8_KERNEL_W8A16_TILE = 12,        /* tiled MFMA kernel, weights widened in registers */
    BFP8_KERNEL_BLK32_STREAM_LDS = 13,  /* block-32, M <= 16: weights through LDS slabs */
    BFP8_KERNEL_BLK32_STREAM = 14,      /* block-32, M > 16 with K split: one 16-token tile per workgroup */
    BFP8_KERNEL_BLK32_GEMV = 15,        /* block-32, one token: dot products on the vector ALUs */
    BFP8_KERNEL_BLK32_WIDE = 16,        /* block-32, M > 8: all tokens of a group per weight tile */
    BFP8_KERNEL_BLK32_TILE = 17,        /* block-32, larger M: tiled MFMA kernel */
    BFP8_KERNEL_COUNT = 18
};

/* A call's launch plan (filled by bfp8_get_plan). */
typedef struct bfp8_plan {
    int32_t kernel;         /* BFP8_KERNEL_* of the op's main kernel */
    int32_t quant_kernel;   /* BFP8_KERNEL_QUANT_ACT when the fused quantise + W8A8 call runs
                               the quantiser as its own launch first, else BFP8_KERNEL_NONE */
    int32_t tile_n;         /* weight rows (output columns) per workgroup tile */
    int32_t tile_m;         /* tokens per workgroup tile, padded (0 for the quantisers) */
    int32_t waves;          /* 64-lane waves per workgroup */
    int32_t splits;         /* workgroups that share one output tile over K (1: K not split) */
    int64_t workgroups;     /* workgroups in the main kernel's grid */
    uint64_t workspace_bytes; /* = bfp8_workspace_bytes(op, M, N, K) */
} bfp8_plan;

/*
 * The launch plan of `op` for an M x N x K problem, from the same routing
 * code the calls use, so a test can state which kernel it exercises and a
 * caller can see the kernel and workspace a shape will get ([ARC]
 * "Correctness guards": what a shape is served by is read from the library,
 * not re-derived by the caller).  Host only, touches no GPU, allocates
 * nothing.  Returns BFP8_E_NULL (plan NULL), BFP8_E_OP (unknown op) or
 * BFP8_E_SHAPE when the call itself would refuse the sizes; `plan` is
 * written only on success.
 */
bfp8_status bfp8_get_plan(int op, int64_t M, int64_t N, int64_t K, bfp8_plan* plan);

/* Static name of a BFP8_KERNEL_* id ("unknown kernel" for others). */
const char* bfp8_kernel_name(int kernel);

/* Static, human-readable text for a status code. */
const char* bfp8_status_string(bfp8_status status);

#ifdef __cplusplus
}
#endif

#endif /* BFP8_H */
