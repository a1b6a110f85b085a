"""Shape tables of the GPU parity tests, each case with the kernel variant it
is meant to exercise.

The GPU tests take their parameters from here and assert, through
bfp8_get_plan, that the library routes each case to the stated kernel.  The
CPU suite (tests/test_plan.py) checks the same routing without a GPU and that
the cases together reach every kernel variant the router can produce, so a
dispatch threshold that moves a case off its kernel, or leaves a kernel with
no parity case, fails the suite.

A variant is the kernel's name; the all-token and tiled kernels add their
workgroup tile and waves (":tile_n x tile_m w waves"), a plan that splits K
adds "/split", and the fused quantise + W8A8 call that stages the codes
through the quantiser first is prefixed "quant+".
"""

import blockwise_scaled_fp8_amd as bfp8

W8A8 = bfp8.OP_GEMM_W8A8_BLK128
QW8A8 = bfp8.OP_QUANT_GEMM_W8A8_BLK128
W8A16 = bfp8.OP_GEMM_W8A16_BLK128
BLK32 = bfp8.OP_GEMM_W8A16_BLK32_UE8M0


def variant(op, M, N, K):
    p = bfp8.bfp8_get_plan(op, M, N, K)
    v = p["kernel_name"]
    if "tile" in v or "wide" in v:
        v += f":{p['tile_n']}x{p['tile_m']}w{p['waves']}"
    if p["splits"] > 1:
        v += "/split"
    if p["quant_kernel"]:
        v = "quant+" + v
    return v


def expect(op, M, N, K, want):
    got = variant(op, M, N, K)
    assert got == want, f"op {op} M={M} N={N} K={K} runs {got}, the case is meant for {want}"


# ------------------------------------------------------------------ W8A8 ----
# Threshold straddle on a small projection (N = 384, K = 640).
W8A8_THRESHOLD = [(1, 384, 640, "w8a8_gemv")] + \
    [(M, 384, 640, "w8a8_stream") for M in (2, 3, 5, 8, 15, 16, 17, 24, 31, 32, 33, 48, 63, 64)] + \
    [(M, 384, 640, "w8a8_wide:16x32w8") for M in (65, 129, 200)]

# One token, K <= 8192: 4 or 8 chunks of 1 KB per lane, K ending inside a
# chunk, one weight row per wave, N of one workgroup up to 12288.
W8A8_ONE_TOKEN = [(1, N, K, "w8a8_gemv") for N, K in
                  ((16, 128), (16, 1152), (64, 4096), (1024, 4096), (2064, 1024), (4096, 3968), (12288, 2048),
                   (512, 4224), (4096, 7168), (2064, 5120), (8192, 8192))]
# Just above the one-token range.
W8A8_ABOVE_ONE_TOKEN = [(1, 512, 8320, "w8a8_stream/split"), (1, 4096, 12416, "w8a8_stream")]

# N not a multiple of 128: tiles straddle weight-scale rows.
W8A8_STRADDLE = [(M, N, 256, "w8a8_stream") for N in (16, 48, 144, 272) for M in (4, 40)]

W8A8_SPLIT_K_STREAM = [(M, 512, 12288, "w8a8_stream/split") for M in (1, 4, 16)]

# Paths that need no workspace for M <= 512 (all-token kernel, or the
# streaming kernel over 16-token tiles on small projections).
W8A8_NO_WORKSPACE = [
    (17, 1024, 4096, "w8a8_stream"), (24, 1024, 4096, "w8a8_stream"), (32, 12288, 12288, "w8a8_wide:64x32w4"),
    (32, 4096, 4096, "w8a8_wide:16x32w8"), (33, 4096, 4096, "w8a8_wide:32x32w8"), (50, 1024, 4096, "w8a8_stream"),
    (64, 4096, 4096, "w8a8_wide:32x32w8"), (32, 12288, 256, "w8a8_wide:64x32w4"), (20, 16, 8192, "w8a8_stream"),
    (20, 8208, 256, "w8a8_wide:64x32w4"),                 # last 64-row weight tile holds 16 rows
    (65, 8192, 512, "w8a8_wide:64x64w4"),
    (100, 4096, 1024, "w8a8_wide:64x32w4"), (128, 1040, 2048, "w8a8_wide:32x32w8"), (20, 64, 128, "w8a8_stream"),
    (128, 8192, 128, "w8a8_wide:64x64w4"),                # one K block: three of the four waves idle
    (64, 1024, 4096, "w8a8_stream"), (40, 2048, 1024, "w8a8_wide:16x32w8"),
    (61, 512, 8192, "w8a8_stream"), (300, 1024, 2048, "w8a8_wide:64x32w4"), (512, 1024, 512, "w8a8_wide:64x32w4"),
    (256, 1040, 1024, "w8a8_wide:64x32w4"), (90, 4096, 1024, "w8a8_wide:32x64w4"),
    (144, 1040, 1024, "w8a8_wide:16x64w4"),               # ragged M and N
    (260, 2064, 1024, "w8a8_wide:64x64w4"),               # ragged M and N (16 rows in the last weight tile)
    (256, 4096, 4096, "w8a8_wide:64x64w4"),
    (1000, 1024, 512, "w8a8_wide:64x64w4"),               # 16 token groups, ragged last group
    # 4 < M <= 16 where streaming would take several rounds of 16-row tiles
    (8, 12288, 1024, "w8a8_wide:64x16w4"), (16, 6160, 2048, "w8a8_wide:32x16w8"),   # ragged N
    (5, 8192, 512, "w8a8_wide:32x16w8"), (12, 16400, 256, "w8a8_stream"),          # no one-round shape
    # 8 < M <= 16 where streaming would leave CUs idle (fewer than 256 weight-row tiles)
    (12, 2064, 1024, "w8a8_wide:16x16w8"), (9, 1024, 6144, "w8a8_wide:16x16w8"), (8, 2048, 4096, "w8a8_stream"),
]

# Long K on the all-token kernel with K split over two or four workgroups
# where the unsplit launch would leave most CUs idle (N <= 1024): ragged M,
# an uneven split (K = 12416: 97 blocks in four parts), K = 16384, one
# token, a single 16-row weight tile.
W8A8_WIDE_SPLIT = [
    (1, 1024, 12288, "w8a8_wide:16x16w8/split"), (5, 1024, 12288, "w8a8_wide:16x16w8/split"),
    (16, 1024, 12288, "w8a8_wide:16x16w8/split"), (11, 1024, 16384, "w8a8_wide:16x16w8/split"),
    (20, 1008, 12416, "w8a8_wide:16x32w8/split"), (32, 1024, 16384, "w8a8_wide:16x32w8/split"),
    (31, 1008, 12288, "w8a8_wide:16x32w8/split"), (17, 16, 12288, "w8a8_wide:16x32w8/split"),
    # 32-row tiles split two ways where 16-row tiles would fill more than 64 workgroups:
    # the down_proj shape, a ragged last tile (N = 1040, 33 tiles), an uneven split (97 blocks) with ragged M
    (32, 4096, 12288, "w8a8_wide:32x32w8/split"), (17, 1040, 12288, "w8a8_wide:32x32w8/split"),
    (25, 4080, 12416, "w8a8_wide:32x32w8/split"),
]

# Every tiled configuration, ragged M and N tiles, split K.
W8A8_TILE = [
    (40, 8192, 8192, "w8a8_tile:128x64w8/split"),
    (65, 1024, 8192, "w8a8_tile:64x128w8/split"),
    (100, 1024, 8192, "w8a8_tile:64x128w8/split"),
    (200, 2048, 4224, "w8a8_tile:64x128w8/split"),        # last split shorter (33 blocks in 4)
    (66, 2064, 8192, "w8a8_tile:64x128w8/split"),         # ragged N and M
    (500, 2064, 1024, "w8a8_tile:64x128w8"),              # ragged N and M, K not split
    (1000, 4096, 1024, "w8a8_tile:128x128w8"),
    (400, 2048, 8192, "w8a8_tile:128x128w8/split"),       # ragged M
    (512, 4096, 8192, "w8a8_tile:128x128w8/split"),
    (2000, 4000, 1024, "w8a8_tile:256x128w8"),            # ragged M and N
    (388, 4112, 512, "w8a8_tile:128x64w8"),               # ragged M and N, K not split
]
W8A8_LARGE_RAGGED = (4000, 4000, 384, "w8a8_tile:256x256w8")
W8A8_DECODE_OPROJ = (1, 4096, 4096, "w8a8_gemv")
W8A8_PREFILL_OPROJ = (4096, 4096, 4096, "w8a8_tile:256x256w8")
W8A8_ONE_HOT = [(1, 256, 256, "w8a8_gemv"), (3, 256, 256, "w8a8_stream"), (48, 256, 256, "w8a8_stream")]
W8A8_DETERMINISTIC = (64, 512, 1024, "w8a8_stream")

# Fused quantise + W8A8 (bit-identical to quantise-then-GEMM).
QUANT_W8A8 = [
    (1, 4096, 4096, "w8a8_gemv_quant"), (1, 16, 128, "w8a8_gemv_quant"), (1, 1024, 1152, "w8a8_gemv_quant"),
    (1, 2064, 3968, "w8a8_gemv_quant"), (1, 512, 4224, "w8a8_gemv_quant"), (1, 4096, 7168, "w8a8_gemv_quant"),
    (1, 512, 8320, "w8a8_stream_quant/split"), (2, 1024, 4096, "w8a8_stream_quant"),
    (3, 512, 640, "w8a8_stream_quant"), (4, 384, 12288, "w8a8_stream_quant/split"),
    (5, 1024, 4096, "w8a8_stream_quant"), (8, 512, 1024, "w8a8_stream_quant"), (9, 512, 640, "quant+w8a8_stream"),
    (16, 1024, 4096, "quant+w8a8_wide:16x16w8"), (17, 384, 640, "quant+w8a8_stream"), (64, 1024, 4096, "quant+w8a8_stream"),
    (300, 1040, 1024, "quant+w8a8_wide:64x32w4"), (200, 2048, 4224, "quant+w8a8_tile:64x128w8/split"),
    (6, 8192, 1024, "quant+w8a8_wide:32x16w8"), (16, 12288, 512, "quant+w8a8_wide:64x16w4"),
]

# ---------------------------------------------------------------- W8A16 ----
W8A16_BY_M = [(1, 512, 1024, "w8a16_gemv")] + \
    [(M, 512, 1024, "w8a16_stream") for M in (2, 3, 4, 5, 8)] + \
    [(M, 512, 1024, "w8a16_wide:16x16w8") for M in (9, 12, 16)] + \
    [(M, 512, 1024, "w8a16_wide:16x32w4") for M in (17, 33, 64, 65, 130)]
# 8 < M <= 16 without a split of K: the all-token kernel with one 16-token
# tile, one or two weight-row tiles (a half-filled pair at N = 16), ragged
# M, K of one block and long K.
W8A16_ONE_TILE = [
    (16, 4096, 4096, "w8a16_wide:16x16w8"), (9, 1024, 4096, "w8a16_wide:16x16w8"),
    (13, 12288, 512, "w8a16_wide:64x16w4"), (16, 16, 4096, "w8a16_wide:16x16w8"), (11, 64, 128, "w8a16_wide:16x16w8"),
    (16, 8176, 512, "w8a16_wide:32x16w8"),                # last 32-row weight tile holds 16 rows
    (12, 8208, 256, "w8a16_wide:64x16w4"),                # last 64-row weight tile holds 16 rows
    # 4 <= M <= 8 where streaming would take several rounds
    (4, 12288, 512, "w8a16_wide:64x16w4"), (8, 8208, 1024, "w8a16_wide:64x16w4"), (3, 12288, 512, "w8a16_stream"),
    (16, 4096, 7168, "w8a16_wide:16x16w8"),
]
# One token, K <= 12288: 4, 8 or 12 chunks, one row per wave.
W8A16_ONE_TOKEN = [(1, N, K, "w8a16_gemv") for N, K in
                   ((16, 128), (16, 1152), (64, 4096), (1024, 4096), (2064, 1024), (4096, 4096), (4096, 3968),
                    (12288, 2048), (2064, 5120), (8192, 8192), (4096, 12288))]
W8A16_ALL_TOKENS = [
    (17, 1024, 4096, "w8a16_wide:16x32w4"), (32, 4096, 4096, "w8a16_wide:16x32w4"),
    (50, 1024, 4096, "w8a16_wide:16x32w4"), (64, 4096, 4096, "w8a16_wide:32x32w4"),
    (24, 12288, 512, "w8a16_wide:64x32w4"), (20, 16, 4096, "w8a16_wide:16x32w4"), (20, 64, 128, "w8a16_wide:16x32w4"),
    (128, 4096, 4096, "w8a16_wide:64x32w4"), (90, 4112, 1024, "w8a16_wide:64x32w4"),   # ragged M and N
    (256, 1024, 4096, "w8a16_wide:32x32w4"), (144, 1040, 1024, "w8a16_wide:16x64w4"),
    (32, 8176, 512, "w8a16_wide:32x32w4"),                # last 32-row weight tile holds 16 rows
    (512, 1024, 4096, "w8a16_wide:64x32w4"), (200, 1040, 1024, "w8a16_wide:32x32w4"),
    (40, 1024, 8192, "w8a16_wide:16x32w4"), (48, 4096, 7168, "w8a16_wide:32x32w4"),
]
W8A16_LONG_K = [(1, 4096, 12416, "w8a16_stream"), (3, 4096, 12288, "w8a16_stream"),
                (16, 4096, 12288, "w8a16_wide:16x16w8")]
# K split over workgroups, also with sixteen live token rows (8 < M <= 16,
# the streaming kernel's register-operand tokens).
W8A16_SPLIT_K_STREAM = [(4, 512, 12288, "w8a16_stream/split"), (12, 512, 12288, "w8a16_stream/split")]
W8A16_ONE_HOT = [(1, 256, 256, "w8a16_gemv"), (4, 256, 256, "w8a16_stream"), (16, 256, 256, "w8a16_wide:16x16w8"),
                 (40, 256, 256, "w8a16_wide:16x32w4")]
W8A16_TILE_SPLIT = [(40, 1024, 12288, "w8a16_tile:128x64w8/split"), (100, 1040, 8192, "w8a16_tile:128x128w8/split"),
                    (300, 2048, 2176, "w8a16_tile:128x128w8/split"), (40, 16384, 512, "w8a16_tile:128x64w8")]
W8A16_TILE_ONE_HOT = (8200, 256, 256, "w8a16_tile:128x128w8")
W8A16_TILE_LARGE_RAGGED = (2000, 4112, 1024, "w8a16_tile:256x128w8")
W8A16_TILE_LARGE_ONE_HOT = (2048, 4096, 256, "w8a16_tile:256x128w8")
W8A16_PREFILL_OPROJ = (4096, 4096, 4096, "w8a16_tile:256x128w8")
W8A16_DECODE_OPROJ = (1, 4096, 4096, "w8a16_gemv")

# ---------------------------------------------------------------- blk32 ----
BLK32_WORKLOAD = [(1, 4096, 7168, "blk32_gemv")] + [(M, 4096, 7168, "blk32_stream_lds") for M in (2, 3, 4, 8)] + \
    [(M, 4096, 7168, "blk32_wide:16x16w8") for M in (9, 12, 16)]
# 8 < M <= 16 without a split of K: the all-token kernel with one 16-token
# tile, the UE8M0 scales applied in the widening; one and two weight-row
# tiles (two: 16 weight rows of each of two 16-row halves of a 32-row scale
# band), ragged M, tiny N.
BLK32_ONE_TILE = [(13, 8192, 1152, "blk32_wide:32x16w8"), (16, 12288, 1024, "blk32_wide:32x16w8"),
                  (10, 64, 4096, "blk32_wide:16x16w8"), (16, 32, 256, "blk32_wide:16x16w8")]
# One token with K <= 8192: the dot-product kernel on the vector ALUs (one and
# 4 or 8 chunks, K of one block and K ending inside a 1 KB chunk), and
# just above that range.
BLK32_ONE_TOKEN = [(1, 4096, 4096, "blk32_gemv"), (1, 32, 128, "blk32_gemv"), (1, 8192, 1152, "blk32_gemv"),
                   (1, 1024, 3968, "blk32_gemv"), (1, 1024, 8192, "blk32_gemv"), (1, 8192, 7168, "blk32_gemv"),
                   (1, 4096, 12416, "blk32_stream_lds")]
BLK32_ONE_HOT_ONE_TOKEN = (1, 704, 256, "blk32_gemv")
# Above the streaming range ([SM70] "Results" times M = 32 ... 4096).
BLK32_ABOVE_16 = [(17, 4096, 7168, "blk32_wide:16x32w4"), (32, 4096, 7168, "blk32_wide:16x32w4"),
                  (32, 8192, 1024, "blk32_wide:32x32w4"), (64, 4096, 2048, "blk32_wide:32x32w4"),
                  (128, 4096, 4096, "blk32_wide:32x64w8"), (100, 1024, 4096, "blk32_wide:16x32w4"),
                  (200, 1024, 1024, "blk32_wide:16x64w4")]
# Larger M: the W8A16 tiled kernel with the UE8M0 scales applied in the
# widening; every tile shape, split and unsplit, ragged M and N (N = 1056
# and 4128: waves of the last weight tile past N read the last scale band).
BLK32_TILE = [(64, 4096, 7168, "blk32_tile:128x64w8/split"), (48, 16384, 512, "blk32_tile:128x64w8"),
              (128, 4096, 7168, "blk32_tile:128x128w8/split"), (300, 1056, 2048, "blk32_tile:128x128w8/split"),
              (600, 256, 256, "blk32_tile:128x128w8"), (2048, 4096, 256, "blk32_tile:256x128w8"),
              (2000, 4128, 512, "blk32_tile:256x128w8")]
BLK32_TILE_ONE_HOT = (300, 704, 256, "blk32_tile:128x128w8")
BLK32_WINDOW = (8, 512, 1024, "blk32_stream_lds")
BLK32_ONE_HOT = (16, 704, 256, "blk32_wide:16x16w8")
BLK32_ONE_HOT_STREAM = (8, 704, 256, "blk32_stream_lds")
BLK32_ONE_HOT_ABOVE_16 = (17, 704, 256, "blk32_wide:16x32w4")
BLK32_ONE_HOT_ABOVE_16_SPLIT = (17, 704, 8320, "blk32_stream/split")
BLK32_SPLIT_K = (4, 1024, 12288, "blk32_stream_lds/split")
BLK32_SPLIT_K_16 = (16, 1024, 12288, "blk32_stream_lds/split")
BLK32_SPLIT_K_ABOVE_16 = (20, 512, 12288, "blk32_stream/split")


# The longest K the calls accept (2^23): every kernel family's 32-bit buffer
# offsets at their largest (weight and token rows 2^23 bytes, or 2^24 for
# 16-bit tokens, apart), with K split across workgroups.
K_MAX = 1 << 23
W8A8_MAX_K = [(3, 32, K_MAX, "w8a8_stream/split"), (20, 64, K_MAX, "w8a8_wide:16x32w8/split"),
              (40, 128, K_MAX, "w8a8_tile:64x128w8/split")]
QUANT_W8A8_MAX_K = [(2, 32, K_MAX, "w8a8_stream_quant/split")]
W8A16_MAX_K = [(3, 32, K_MAX, "w8a16_stream/split"), (40, 128, K_MAX, "w8a16_tile:128x64w8/split")]
BLK32_MAX_K = [(1, 32, K_MAX, "blk32_stream_lds/split"), (40, 64, K_MAX, "blk32_stream/split")]


def coverage_key(op, v):
    """The fused call that stages the codes through the quantiser runs the
    same W8A8 kernel as the codes call: its variants count as that call's
    (a separate check asks for at least one staged case)."""
    if op == QW8A8 and v.startswith("quant+"):
        return (W8A8, v[len("quant+"):])
    return (op, v)


def all_cases():
    """(op, M, N, K, variant) for every case above."""
    out = []
    tables = {
        W8A8: [W8A8_THRESHOLD, W8A8_ONE_TOKEN, W8A8_ABOVE_ONE_TOKEN, W8A8_STRADDLE, W8A8_SPLIT_K_STREAM, W8A8_NO_WORKSPACE,
               W8A8_WIDE_SPLIT, W8A8_TILE,
               [W8A8_LARGE_RAGGED, W8A8_DECODE_OPROJ, W8A8_PREFILL_OPROJ, W8A8_DETERMINISTIC], W8A8_ONE_HOT,
               W8A8_MAX_K],
        QW8A8: [QUANT_W8A8, QUANT_W8A8_MAX_K],
        W8A16: [W8A16_BY_M, W8A16_ONE_TOKEN, W8A16_ONE_TILE, W8A16_ALL_TOKENS, W8A16_LONG_K, W8A16_SPLIT_K_STREAM,
                W8A16_ONE_HOT,
                W8A16_TILE_SPLIT, [W8A16_TILE_ONE_HOT, W8A16_TILE_LARGE_RAGGED, W8A16_TILE_LARGE_ONE_HOT,
                                   W8A16_PREFILL_OPROJ, W8A16_DECODE_OPROJ], W8A16_MAX_K],
        BLK32: [BLK32_WORKLOAD, BLK32_ONE_TOKEN, BLK32_ONE_TILE, BLK32_ABOVE_16, BLK32_TILE, [BLK32_TILE_ONE_HOT],
                [BLK32_WINDOW, BLK32_ONE_HOT, BLK32_ONE_HOT_STREAM, BLK32_ONE_HOT_ABOVE_16,
                 BLK32_ONE_HOT_ABOVE_16_SPLIT, BLK32_ONE_HOT_ONE_TOKEN,
                 BLK32_SPLIT_K, BLK32_SPLIT_K_16, BLK32_SPLIT_K_ABOVE_16], BLK32_MAX_K],
    }
    for op, tabs in tables.items():
        for tab in tabs:
            for (M, N, K, v) in tab:
                out.append((op, M, N, K, v))
    return out
