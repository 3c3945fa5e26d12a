"""Pins for the oracle's shard-range rule (CPU only)."""
import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_walkthrough_inner_split_is_3_then_2():
    g = json.load(open(os.path.join(GOLDEN, "walkthrough_shapes.json")))
    ranges = oracle.shard_ranges(g["K"], g["parts"])
    assert [hi - lo for lo, hi in ranges] == g["inner_split_sizes"]
    assert ranges[0][0] == 0 and ranges[-1][1] == g["K"]


@pytest.mark.parametrize("n", range(0, 65))
def test_matches_numpy_array_split(n):
    # np.array_split is an independent library routine with the same
    # larger-shards-first contiguous rule.
    for parts in range(1, 71):
        pieces = np.array_split(np.arange(n), parts)
        got = oracle.shard_ranges(n, parts)
        assert len(got) == parts
        for (lo, hi), piece in zip(got, pieces):
            assert hi - lo == len(piece)
            if len(piece):
                assert (lo, hi) == (int(piece[0]), int(piece[-1]) + 1)


def test_partition_properties():
    rng = np.random.default_rng(1)
    for _ in range(500):
        n = int(rng.integers(0, 10_000))
        parts = int(rng.integers(1, 300))
        r = oracle.shard_ranges(n, parts)
        sizes = [hi - lo for lo, hi in r]
        assert sum(sizes) == n
        assert all(r[i][1] == r[i + 1][0] for i in range(parts - 1))
        assert max(sizes) - min(sizes) <= 1
        assert sizes == sorted(sizes, reverse=True)
        if parts > n:
            assert sizes.count(0) == parts - n


def test_divisible_equals_equal_chunks():
    # TP lesson page solution slices i*chunk:(i+1)*chunk when tp divides the dim.
    for n, p in [(256, 4), (128256, 8), (14336, 8), (28672, 8), (8192, 8)]:
        c = n // p
        assert oracle.shard_ranges(n, p) == [(i * c, (i + 1) * c) for i in range(p)]


@pytest.mark.parametrize("bad", [0, -1, 2.0, True, "2"])
def test_bad_parts_raise_partition(bad):
    with pytest.raises(ValueError, match="partition"):
        oracle.shard_ranges(5, bad)


def test_bad_rank_raises():
    with pytest.raises(ValueError, match="partition"):
        oracle.shard_range(5, 2, 2)
    with pytest.raises(ValueError, match="shape"):
        oracle.shard_range(-1, 2, 0)
