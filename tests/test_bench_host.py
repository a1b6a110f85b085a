"""Host-side logic of bench.py, on the CPU: the weight rotation never lets a
timed launch find its weights in the 256 MiB last-level cache, for the
short runs (--steps 20 --warmup 5) and the defaults, and the reuse check catches a rotation
that does."""

import pytest

import bench

MIB = 1 << 20


@pytest.mark.parametrize("steps,warmup", [(20, 5), (200, 20), (7, 0), (1000, 100)])
def test_decode_rotation_leaves_the_cache_cold(steps, warmup):
    C = 24                                  # the default --copies
    seq, timed = bench.launch_order(["w8", "w16"], {"w8": lambda i: i % C, "w16": lambda i: i % C}, warmup, steps)
    d = bench.assert_no_cache_reuse((seq, timed), {"w8": 16 * MIB, "w16": 16 * MIB}, "decode")
    assert d is None or d >= 256 * MIB


def test_reuse_check_catches_a_short_rotation():
    # the previous layout: one shared set of 32 copies, W8A16 offset by half a set
    C = 32
    seq, timed = bench.launch_order(["a", "b"], {"a": lambda i: i % C, "b": lambda i: (i + C // 2) % C}, 5, 20)
    seq = [("w", c) for _, c in seq]        # both kernels read the same copies
    with pytest.raises(AssertionError):
        bench.assert_no_cache_reuse((seq, timed), {"w": 16 * MIB}, "shared set")


def test_reuse_distance_counts_bytes_between_reads():
    seq = [("a", 0), ("a", 1), ("a", 2), ("a", 0)]
    assert bench.min_reuse_bytes(seq, {"a": 10}) == 20
    assert bench.min_reuse_bytes(seq, {"a": 10}, first=4) is None


def test_block32_extra_rotation():
    seq, timed = bench.launch_order(["g"], {"g": lambda i: i % 12}, 20, 200)
    assert bench.assert_no_cache_reuse((seq, timed), {"g": 4096 * 7168}, "block-32") >= 256 * MIB
