"""Pins for the oracle pack / unpack.

The expected home buffers are built independently of the oracle's offset
arithmetic: full matrices are made first, cut into per-shard row blocks with
``np.split`` at cumulative row boundaries, and the shards are then the
per-shard concatenations. Pack must give back the full matrices, grouped per
home in increasing index order.
"""

import json
import os

import numpy as np
import pytest

from oracle import planner, route

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _make_shards(fulls, split_rows, S):
    shards = [[] for _ in range(S)]
    for f, split in zip(fulls, split_rows):
        blocks = np.split(f, np.cumsum(split)[:-1], axis=0)
        for s in range(S):
            shards[s].append(blocks[s].ravel())
    return [np.concatenate(p) if p else np.zeros(0, np.uint16) for p in shards]


def _expected_homes(fulls, home, S):
    out = []
    for h in range(S):
        parts = [f.ravel() for i, f in enumerate(fulls) if home[i] == h]
        out.append(np.concatenate(parts) if parts else np.zeros(0, np.uint16))
    return out


def test_worked_example_pack():
    with open(os.path.join(GOLDEN, "owner_gather_example.json")) as f:
        ex = json.load(f)
    shapes = ex["printed"]["shapes"]
    split = ex["derived_by_hand"]["split_rows"]
    owners = [1, 1]
    # global flat buffer of 40 elements (iota), split evenly over 2 ranks
    flat = np.arange(40, dtype=np.float32)
    shards = [flat[0:20], flat[20:40]]
    homes = route.pack(shards, shapes, split, owners, 2)
    assert homes[0].size == 0
    assert homes[1].size == 40
    # param_0 = the 20 elements from rank 0 followed by rank 1's own 4
    assert np.array_equal(homes[1][0:20], shards[0][0:20])
    assert np.array_equal(homes[1][20:24], shards[1][0:4])
    # param_1 = rank 1's own 16 elements
    assert np.array_equal(homes[1][24:40], shards[1][4:20])
    back = route.unpack(homes, shapes, split, owners, 2)
    assert all(np.array_equal(a, b) for a, b in zip(back, shards))


@pytest.mark.parametrize("seed", range(12))
def test_pack_matches_independent_construction(seed):
    rng = np.random.default_rng(seed)
    S = int(rng.integers(1, 6))
    n = int(rng.integers(1, 9))
    shapes, fulls, split_rows = [], [], []
    for i in range(n):
        nd = int(rng.integers(2, 4))
        dims = [int(rng.integers(0 if i == 0 else 1, 9))] + [int(rng.integers(1, 6)) for _ in range(nd - 1)]
        shapes.append(tuple(dims))
        P = dims[0]
        f = rng.integers(0, 65535, size=(P, int(np.prod(dims[1:]))), dtype=np.uint16)
        fulls.append(f)
        # random split with zeros
        cuts = np.sort(rng.integers(0, P + 1, size=S - 1))
        split = np.diff(np.concatenate([[0], cuts, [P]])).astype(int).tolist()
        split_rows.append(split)
    home = [int(rng.integers(0, S)) for _ in range(n)]
    shards = _make_shards(fulls, split_rows, S)
    homes = route.pack(shards, shapes, split_rows, home, S)
    expected = _expected_homes(fulls, home, S)
    for h in range(S):
        assert np.array_equal(homes[h], expected[h])
    # full_matrix views recover each tensor in its shape
    for i in range(n):
        m = route.full_matrix(homes, shapes, split_rows, home, S, i)
        assert np.array_equal(m.reshape(fulls[i].shape), fulls[i])
    back = route.unpack(homes, shapes, split_rows, home, S)
    for s in range(S):
        assert np.array_equal(back[s], shards[s])


def test_single_shard_is_identity_copy():
    # a trivial group (size 1) moves nothing: pack is a plain copy
    rng = np.random.default_rng(7)
    shapes = [(3, 4), (5, 2), (1, 9)]
    flat = rng.integers(0, 1000, size=sum(a * b for a, b in shapes)).astype(np.uint16)
    homes = route.pack([flat], shapes, [[3], [5], [1]], [0, 0, 0], 1)
    assert np.array_equal(homes[0], flat)


def test_offsets_reject_bad_split():
    with pytest.raises(ValueError):
        planner.route_offsets([(4, 2)], [[1, 1]], [0], 2)
