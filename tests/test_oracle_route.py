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


def _random_axis_case(rng, S, n):
    shapes, fulls, split, dims = [], [], [], []
    for _ in range(n):
        nd = int(rng.integers(2, 5))
        shape = tuple(int(rng.integers(0, 6)) for _ in range(nd))
        d = int(rng.integers(0, nd))
        cuts = np.sort(rng.integers(0, shape[d] + 1, size=S - 1))
        split.append(np.diff(np.concatenate([[0], cuts, [shape[d]]])).astype(int).tolist())
        shapes.append(shape)
        dims.append(d)
        fulls.append(rng.integers(0, 65535, size=shape, dtype=np.uint16))
    return shapes, fulls, split, dims


@pytest.mark.parametrize("seed", range(10))
def test_pack_axis_matches_split_construction_and_brute_force(seed):
    rng = np.random.default_rng(900 + seed)
    S = int(rng.integers(1, 5))
    n = int(rng.integers(1, 7))
    shapes, fulls, split, dims = _random_axis_case(rng, S, n)
    home = [int(rng.integers(0, S)) for _ in range(n)]
    # shards built with np.split along each tensor's axis
    shards = [[] for _ in range(S)]
    for f, sp, d in zip(fulls, split, dims):
        for s, blk in enumerate(np.split(f, np.cumsum(sp)[:-1], axis=d)):
            shards[s].append(blk.ravel())
    shards = [np.concatenate(p) if p else np.zeros(0, np.uint16) for p in shards]
    homes = route.pack_axis(shards, shapes, split, dims, home, S)
    for h in range(S):
        want = [fulls[i].ravel() for i in range(n) if home[i] == h]
        assert np.array_equal(homes[h], np.concatenate(want) if want else np.zeros(0, np.uint16))
    # brute force: walk every element of every shard slice with plain index arithmetic
    cursor = [0] * S
    hpos = {}
    for h in range(S):
        pos = 0
        for i in range(n):
            if home[i] == h:
                hpos[i] = pos
                pos += int(np.prod(shapes[i]))
    for i in range(n):
        shape, d = shapes[i], dims[i]
        lo = 0
        for s in range(S):
            w = split[i][s]
            sub = list(shape)
            sub[d] = w
            for flat_sub, idx in enumerate(np.ndindex(*sub)):
                full_idx = list(idx)
                full_idx[d] += lo
                flat_full = int(np.ravel_multi_index(full_idx, shape))
                assert homes[home[i]][hpos[i] + flat_full] == shards[s][cursor[s] + flat_sub]
            cursor[s] += int(np.prod(sub))
            lo += w
    back = route.unpack_axis(homes, shapes, split, dims, home, S)
    assert all(np.array_equal(a, b) for a, b in zip(back, shards))


def test_pack_axis_dim0_equals_row_pack():
    rng = np.random.default_rng(5)
    S, n = 3, 5
    shapes = [(int(rng.integers(1, 9)), int(rng.integers(1, 6))) for _ in range(n)]
    split = []
    for s in shapes:
        cuts = np.sort(rng.integers(0, s[0] + 1, size=S - 1))
        split.append(np.diff(np.concatenate([[0], cuts, [s[0]]])).astype(int).tolist())
    fulls = [rng.integers(0, 65535, size=s, dtype=np.uint16) for s in shapes]
    shards = _make_shards(fulls, split, S)
    home = [2, 0, 0, 1, 2]
    a = route.pack(shards, shapes, split, home, S)
    b = route.pack_axis(shards, shapes, split, [0] * n, home, S)
    assert all(np.array_equal(x, y) for x, y in zip(a, b))


def test_two_stage_rows_then_columns():
    # layer_sharded_a2a page: one exchange over the GTP_remat group along dim 0,
    # then one over the TP group along partition_dim. A tensor cut into an
    # R x C grid of blocks (R row groups, C column groups) is rebuilt by packing
    # the R row blocks of each column group (dim 0), then the C column blocks (dim 1).
    rng = np.random.default_rng(11)
    P, Q, R, C = 7, 9, 3, 2
    full = rng.integers(0, 65535, size=(P, Q), dtype=np.uint16)
    rsplit, csplit = [3, 0, 4], [5, 4]
    rows = np.split(full, np.cumsum(rsplit)[:-1], axis=0)
    # stage 1: within column group t, the R ranks hold (rows_r, cols_t) blocks
    stage1 = []
    for t, cb in enumerate(np.split(np.arange(Q), np.cumsum(csplit)[:-1])):
        shards = [rows[r][:, cb].ravel() for r in range(R)]
        homes = route.pack_axis(shards, [(P, len(cb))], [rsplit], [0], [0], R)
        stage1.append(homes[0])
    # stage 2: the C column blocks, now complete in rows, gathered along dim 1
    homes = route.pack_axis(stage1, [(P, Q)], [csplit], [1], [1], C)
    assert np.array_equal(homes[1].reshape(P, Q), full)


@pytest.mark.parametrize("seed", range(12))
def test_route_offsets_axis_locate_every_piece(seed):
    # Pin for planner.route_offsets with a per-tensor shard_dim, built without
    # its offset arithmetic: every element of every tensor carries a unique
    # tag; shard buffers are the per-shard concatenations of np.split blocks
    # along each tensor's axis, home buffers the per-home concatenations of the
    # whole tensors in index order. Each returned offset must then point at
    # exactly its piece, and the sizes must be the buffers' lengths.
    rng = np.random.default_rng(1700 + seed)
    S = int(rng.integers(1, 6))
    n = int(rng.integers(1, 8))
    shapes, fulls, split, dims = [], [], [], []
    tag = 0
    for i in range(n):
        nd = int(rng.integers(2, 5))
        shape = tuple(int(rng.integers(0 if i == 0 else 1, 6)) for _ in range(nd))
        d = int(rng.integers(0, nd))
        cuts = np.sort(rng.integers(0, shape[d] + 1, size=S - 1))
        split.append(np.diff(np.concatenate([[0], cuts, [shape[d]]])).astype(int).tolist())
        size = int(np.prod(shape))
        fulls.append(np.arange(tag, tag + size, dtype=np.int64).reshape(shape))
        tag += size
        shapes.append(shape)
        dims.append(d)
    home = [int(rng.integers(0, S)) for _ in range(n)]
    blocks = [np.split(f, np.cumsum(sp)[:-1], axis=d) for f, sp, d in zip(fulls, split, dims)]
    shards = [np.concatenate([blocks[i][s].ravel() for i in range(n)]) for s in range(S)]
    homes = []
    for h in range(S):
        parts = [fulls[i].ravel() for i in range(n) if home[i] == h]
        homes.append(np.concatenate(parts) if parts else np.zeros(0, np.int64))
    got = planner.route_offsets(shapes, split, home, S, shard_dim=dims)
    assert got["shard_elems"] == [len(b) for b in shards]
    assert got["home_elems"] == [len(b) for b in homes]
    for i in range(n):
        hb, ho, size = homes[home[i]], got["home_offset"][i], fulls[i].size
        assert np.array_equal(hb[ho:ho + size], fulls[i].ravel())
        lo = 0
        for s in range(S):
            blk = blocks[i][s].ravel()
            so = got["shard_offset"][i][s]
            assert np.array_equal(shards[s][so:so + blk.size], blk)
            assert got["row_start"][i][s] == lo
            lo += split[i][s]


def test_route_offsets_axis_hand_case():
    # a (2, 3, 4) tensor cut along dim 1 as [1, 2] and a (4, 2) tensor cut along
    # dim 0 as [3, 1]: shard 0 holds 2*1*4 = 8 then 3*2 = 6 elements, shard 1
    # holds 2*2*4 = 16 then 1*2 = 2; both tensors homed on 1 (24 then 8).
    got = planner.route_offsets([(2, 3, 4), (4, 2)], [[1, 2], [3, 1]], [1, 1], 2, shard_dim=[1, 0])
    assert got["shard_offset"] == [[0, 0], [8, 16]]
    assert got["shard_elems"] == [14, 18]
    assert got["home_offset"] == [0, 24]
    assert got["home_elems"] == [0, 32]
    assert got["row_start"] == [[0, 1], [0, 3]]
