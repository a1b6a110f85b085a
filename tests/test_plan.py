"""The launch-plan query and the coverage of the GPU parity cases, on the CPU.

bfp8_get_plan reports the kernel, tile, waves, K splits, grid and workspace
the library will use for a shape, from the same routing code as the calls.
These tests check, without a GPU:
  * every GPU parity case (tests/cases.py) still routes to the kernel variant
    it is meant to exercise;
  * every kernel variant that any shape of a broad sweep can reach is
    exercised by at least one GPU parity case;
  * the plan agrees with bfp8_workspace_bytes and with the calls' shape rules.
"""

import itertools

import pytest

import blockwise_scaled_fp8_amd as bfp8
from tests import cases

OPS = (cases.W8A8, cases.QW8A8, cases.W8A16, cases.BLK32)
SWEEP_M = sorted(set(list(range(1, 21)) + [24, 31, 32, 33, 34, 40, 48, 63, 64, 65, 96, 100, 128, 129, 192, 200, 256,
                                           300, 384, 400, 512, 640, 768, 1000, 1024, 1536, 2000, 2048, 3072, 4096, 8192]))
SWEEP_N = [16, 32, 48, 64, 128, 256, 384, 512, 1024, 1040, 2048, 2064, 4096, 4112, 8192, 12288, 16384, 32768]
SWEEP_K = [128, 256, 512, 640, 1024, 2048, 2176, 4096, 4224, 7168, 8192, 12288, 16384]


def _sweep():
    for op, M, N, K in itertools.product(OPS, SWEEP_M, SWEEP_N, SWEEP_K):
        if op == cases.BLK32 and N % 32:
            continue
        yield op, M, N, K


@pytest.mark.parametrize("case", cases.all_cases(), ids=lambda c: f"op{c[0]}-M{c[1]}-N{c[2]}-K{c[3]}")
def test_case_routes_to_its_kernel(case):
    op, M, N, K, want = case
    cases.expect(op, M, N, K, want)


def test_every_reachable_kernel_variant_has_a_parity_case():
    reachable = {}
    for op, M, N, K in _sweep():
        reachable.setdefault(cases.coverage_key(op, cases.variant(op, M, N, K)), (M, N, K))
    covered = {cases.coverage_key(op, v) for op, M, N, K, v in cases.all_cases()}
    missing = {k: reachable[k] for k in reachable if k not in covered}
    assert not missing, f"kernel variants with no GPU parity case (op, variant): example shape {missing}"
    staged = [c for c in cases.all_cases() if c[4].startswith("quant+")]
    assert any("/split" in c[4] for c in staged) and any("/split" not in c[4] for c in staged)
    # and the sweep reaches every kernel id the router knows of
    ids = {bfp8.bfp8_get_plan(op, M, N, K)["kernel"] for op, M, N, K in _sweep()}
    assert ids == set(range(3, 18)), sorted(ids)


def test_plan_agrees_with_workspace_bytes_and_grid():
    for op, M, N, K in _sweep():
        p = bfp8.bfp8_get_plan(op, M, N, K)
        assert p["workspace_bytes"] == bfp8.bfp8_workspace_bytes(op, M, N, K), (op, M, N, K)
        assert p["workgroups"] >= 1 and p["splits"] >= 1 and p["waves"] in (4, 8, 16)
        assert p["tile_n"] >= 1 and p["tile_m"] >= 1
        if p["splits"] > 1:
            assert p["workspace_bytes"] > 0, (op, M, N, K, p)
        if op == cases.QW8A8 and p["quant_kernel"]:
            # the staged codes (M*K bytes) live in the workspace
            assert p["workspace_bytes"] >= M * K


def test_routing_rules_read_off_the_plan():
    """Rules the header states, checked over the sweep."""
    # One token: W8A8 (codes and fused) and block-32 up to K = 8192, W8A16 up to 12288.
    one_token_k = {cases.W8A8: 8192, cases.QW8A8: 8192, cases.W8A16: 12288, cases.BLK32: 8192}
    for op, M, N, K in _sweep():
        name = bfp8.bfp8_get_plan(op, M, N, K)["kernel_name"]
        one = M == 1 and K <= one_token_k[op]
        if op in (cases.W8A8, cases.QW8A8, cases.W8A16):
            assert ("gemv" in name) == one, (op, M, N, K, name)
        if op in (cases.W8A16, cases.BLK32) and M <= 16 and not one:
            # 8 < M <= 16: one token tile on the all-token kernel unless the
            # streaming plan splits K; M <= 8 streams, except W8A16 at
            # 4 <= M <= 8 with K <= 4096 where streaming would take several
            # rounds (over 256 16-row tiles) and the all-token launch fits one.
            p = bfp8.bfp8_get_plan(op, M, N, K)
            stream = "w8a16_stream" if op == cases.W8A16 else "blk32_stream_lds"
            wide = "w8a16_wide" if op == cases.W8A16 else "blk32_wide"
            if M <= 8 and name == wide:
                assert op == cases.W8A16 and M >= 4 and K <= 4096 and N > 16 * 256, (op, M, N, K, p)
                assert p["tile_m"] == 16 and p["workgroups"] <= 256 and p["workspace_bytes"] == 0, (op, M, N, K, p)
            elif M <= 8:
                assert name == stream, (op, M, N, K, name)
            elif name == wide:
                assert p["tile_m"] == 16 and p["workspace_bytes"] == 0, (op, M, N, K, p)
            else:
                assert name == stream and p["splits"] > 1, (op, M, N, K, p)
        if op == cases.BLK32 and (one or M > 16):
            p = bfp8.bfp8_get_plan(op, M, N, K)
            short_k = K <= 4096 and (M <= 32 or (M <= 256 and M * N <= 1 << 19))
            if one:
                assert name == "blk32_gemv", (M, N, K, name)
            elif name == "blk32_stream":
                assert p["splits"] > 1, (M, N, K, p)   # only where the streaming plan splits K
            elif name == "blk32_wide":
                # the all-token kernel: K <= 4096 as for W8A16, or K <= 8192, M <= 32 in one round
                assert p["workspace_bytes"] == 0, (M, N, K, p)
                assert short_k or (K <= 8192 and M <= 32 and p["workgroups"] <= 256), (M, N, K, p)
            else:
                assert name == "blk32_tile" and not short_k, (M, N, K, p)
        if op == cases.QW8A8 and name.endswith("_quant"):
            assert M == 1 or M <= 8


def test_all_token_shapes_follow_their_rules():
    """The all-token shape rules the launch header states, over the sweep:
    one token tile up to 16 tokens; W8A8 past M * N = 2^19 (K <= 4096, M >
    32) only in one round with N >= 512; a K split only at K >= 12288 for
    M <= 32, where one workgroup per weight tile would leave at least three
    quarters of the CUs idle, or, for 16 < M <= 32, as 32-row tiles split two
    ways in place of more than 64 16-row tiles, and always in one round;
    W8A16 blk128 without
    the (4, 4) and (2, 4) forms; block-32 at most two weight-row tiles."""
    for op, M, N, K in _sweep():
        p = bfp8.bfp8_get_plan(op, M, N, K)
        name = p["kernel_name"]
        if not name.endswith("_wide"):
            continue
        kr, kt = p["tile_n"] // 16, p["tile_m"] // 16
        where = (op, M, N, K, p)
        assert kr in (1, 2, 4) and kt in (1, 2, 4), where
        assert (kt == 1) == (M <= 16), where
        # (the fused call's workspace also holds the staged codes)
        assert op == cases.QW8A8 or p["workspace_bytes"] == 0 or p["splits"] > 1, where
        if name == "w8a8_wide":
            if M > 32 and M * N > 1 << 19:
                assert K <= 4096 and N >= 512 and p["workgroups"] <= 256, where
            if p["splits"] > 1:
                assert K >= 12288 and M <= 32 and p["splits"] in (2, 4), where
                assert p["workgroups"] <= 256, where
                if p["workgroups"] // p["splits"] > 64:
                    # 32-row tiles split two ways in place of 16-row tiles on more than 64 workgroups
                    assert (kr, kt, p["splits"]) == (2, 2, 2) and M > 16, where
                    assert (N + 15) // 16 > 64 and p["workgroups"] >= (N + 15) // 16, where
                assert (K // 128) // p["splits"] >= 24 and p["workspace_bytes"] > 0, where
                if op == cases.W8A8:
                    assert p["workspace_bytes"] == 256 * ((p["workgroups"] // p["splits"] * 4 + 255) // 256) + \
                        p["workgroups"] * kr * kt * 256 * 4, where
            assert p["waves"] == (4 if kr == 4 or kt == 4 else 8), where
        elif name == "w8a16_wide":
            assert p["splits"] == 1 and (kr, kt) not in ((4, 4), (2, 4)), where
            assert p["waves"] == (4 if kr == 4 or (kt > 1 and not (kt == 4 and kr == 2)) else 8), where
        else:
            assert name == "blk32_wide" and kr <= 2 and p["splits"] == 1, where


def test_plan_refusals():
    p = bfp8.bfp8_get_plan(cases.W8A8, 1, 4096, 4096)
    assert p["kernel_name"] == "w8a8_gemv"
    for op, M, N, K in [(cases.W8A8, 0, 4096, 4096), (cases.W8A8, 4, 4100, 4096), (cases.W8A8, 4, 4096, 4000),
                        (cases.BLK32, 4, 4112, 7168), (cases.W8A16, 4, 4096, 64), (cases.QW8A8, -1, 16, 128)]:
        with pytest.raises(bfp8.Bfp8Error) as e:
            bfp8.bfp8_get_plan(op, M, N, K)
        assert e.value.name == "BFP8_E_SHAPE"
    with pytest.raises(bfp8.Bfp8Error) as e:
        bfp8.bfp8_get_plan(99, 1, 16, 128)
    assert e.value.name == "BFP8_E_OP"
    lib = bfp8.load()
    assert lib.bfp8_get_plan(cases.W8A8, 1, 16, 128, None) == 1      # BFP8_E_NULL


def test_quantiser_plans():
    p = bfp8.bfp8_get_plan(bfp8.OP_QUANT_ACT_1X128, 4096, 0, 4096)
    assert p["kernel_name"] == "quant_act_1x128" and p["workgroups"] >= 1
    p = bfp8.bfp8_get_plan(bfp8.OP_QUANT_WEIGHT_128X128, 0, 4096, 4096)
    assert p["kernel_name"] == "quant_weight_128x128" and p["workgroups"] == 32 * 32


def test_kernel_names():
    names = [bfp8.bfp8_kernel_name(k) for k in range(18)]
    assert len(set(names)) == 18 and "unknown kernel" not in names
    assert bfp8.bfp8_kernel_name(99) == "unknown kernel"
