"""Oracle pack / unpack: gather row shards into full matrices at their homes and
scatter full results back into the shards.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``). Bit copies with NumPy
slicing and concatenation; works on any dtype (bf16 is carried as uint16).
"""

from __future__ import annotations

import numpy as np

from . import planner


def pack(shard_bufs, shapes, split_rows, home, num_shards: int):
    """Forward routing: every home gets its complete (P, Q) matrices.

    layer_sharded_a2a page, ``route_to_ns_home``: each rank holds a row shard of
    every param, and each home ends up with the complete matrices of the params
    assigned to it, in increasing index order. owner_planning page,
    ``OwnerGatherPlan.reconstruct_full``: a full tensor is the concatenation of
    the per-rank shards in buffer order.

    shard_bufs: list of S flat arrays laid out as in planner.route_offsets.
    Returns a list of S flat arrays (empty for homes with no params).

    Pinned by: the worked example and a per-element brute-force map
    (tests/test_oracle_route.py).
    """
    off = planner.route_offsets(shapes, split_rows, home, num_shards)
    groups = planner.params_by_home(len(shapes), home, num_shards)
    dtype = shard_bufs[0].dtype if num_shards else np.uint16
    homes = []
    for h in range(num_shards):
        parts = []
        for i in groups[h]:
            _, cols = planner.matrix_view(shapes[i])
            for s in range(num_shards):
                start = off["shard_offset"][i][s]
                parts.append(shard_bufs[s][start:start + split_rows[i][s] * cols])
        homes.append(np.concatenate(parts) if parts else np.zeros(0, dtype=dtype))
    return homes


def unpack(home_bufs, shapes, split_rows, home, num_shards: int):
    """Backward routing: every shard gets its rows of every result back.

    layer_sharded_a2a page, ``route_from_ns_home``: every rank receives its row
    shard of every param's result. owner_planning page,
    ``OwnerScatterPlan.unpack``: destinations extract their flat result shards.

    Returns a list of S flat arrays laid out as in planner.route_offsets.

    Pinned by: unpack(pack(x)) == x over random splits, and the brute-force map.
    """
    off = planner.route_offsets(shapes, split_rows, home, num_shards)
    dtype = home_bufs[0].dtype if num_shards else np.uint16
    shards = []
    for s in range(num_shards):
        parts = []
        for i in range(len(shapes)):
            rows, cols = planner.matrix_view(shapes[i])
            h = home[i]
            full = home_bufs[h][off["home_offset"][i]:off["home_offset"][i] + rows * cols]
            r0 = off["row_start"][i][s]
            parts.append(full[r0 * cols:(r0 + split_rows[i][s]) * cols])
        shards.append(np.concatenate(parts) if parts else np.zeros(0, dtype=dtype))
    return shards


def full_matrix(home_bufs, shapes, split_rows, home, num_shards: int, i: int):
    """View of tensor i's complete matrix inside its home buffer, in its shape."""
    off = planner.route_offsets(shapes, split_rows, home, num_shards)
    rows, cols = planner.matrix_view(shapes[i])
    h = home[i]
    flat = home_bufs[h][off["home_offset"][i]:off["home_offset"][i] + rows * cols]
    return flat.reshape(tuple(shapes[i]))


def _slice_shape(shape, dim: int, width: int):
    s = list(shape)
    s[dim] = width
    return tuple(s)


def pack_axis(shard_bufs, shapes, split_sizes, shard_dim, home, num_shards: int):
    """Forward routing with shards cut along any dimension.

    layer_sharded_a2a page, ``route_to_ns_home``: the helper is axis-generic,
    ``shard_dim`` naming the dimension the shards split (0 for the GTP_remat
    stage, the param's partition_dim for the TP stage). Shard buffer s holds,
    for every tensor i in increasing index order, the slice of tensor i along
    shard_dim[i] of width split_sizes[i][s] (the slices follow each other along
    that dimension in buffer order), flattened row-major. A home gets the
    complete tensor: the slices concatenated along shard_dim in buffer order,
    tensors in increasing index order (``params_by_home``).

    Pinned by: equality with ``pack`` for shard_dim 0, a construction with
    ``np.split`` along the axis, a per-element brute-force map, and the
    two-stage (rows, then columns) composition (tests/test_oracle_route.py).
    """
    n = len(shapes)
    dtype = shard_bufs[0].dtype if num_shards else np.uint16
    cursor = [0] * num_shards
    fulls = []
    for i in range(n):
        shape, d = tuple(shapes[i]), shard_dim[i]
        if sum(split_sizes[i]) != shape[d]:
            raise ValueError(f"split sizes of tensor {i} do not sum to dim {d}")
        blocks = []
        for s in range(num_shards):
            sub = _slice_shape(shape, d, split_sizes[i][s])
            cnt = int(np.prod(sub))
            blocks.append(shard_bufs[s][cursor[s]:cursor[s] + cnt].reshape(sub))
            cursor[s] += cnt
        fulls.append(np.concatenate(blocks, axis=d).ravel())
    groups = planner.params_by_home(n, home, num_shards)
    return [np.concatenate([fulls[i] for i in groups[h]]) if groups[h] else np.zeros(0, dtype=dtype)
            for h in range(num_shards)]


def unpack_axis(home_bufs, shapes, split_sizes, shard_dim, home, num_shards: int):
    """Backward routing with shards cut along any dimension: the inverse of
    ``pack_axis`` (layer_sharded_a2a page, ``route_from_ns_home``, and the
    owner_planning page's ``OwnerScatterPlan.unpack``): each shard gets, per
    tensor in index order, its slice along shard_dim of the home's result.

    Pinned by: unpack_axis(pack_axis(x)) == x and the brute-force map.
    """
    n = len(shapes)
    dtype = home_bufs[0].dtype if num_shards else np.uint16
    groups = planner.params_by_home(n, home, num_shards)
    start = {}
    for h in range(num_shards):
        pos = 0
        for i in groups[h]:
            start[i] = pos
            pos += int(np.prod(shapes[i]))
    parts = [[] for _ in range(num_shards)]
    for i in range(n):
        shape, d = tuple(shapes[i]), shard_dim[i]
        numel = int(np.prod(shape))
        full = home_bufs[home[i]][start[i]:start[i] + numel].reshape(shape)
        for s, blk in enumerate(np.split(full, np.cumsum(split_sizes[i])[:-1], axis=d)):
            parts[s].append(blk.ravel())
    return [np.concatenate(p) if p else np.zeros(0, dtype=dtype) for p in parts]
