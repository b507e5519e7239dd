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
