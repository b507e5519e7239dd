"""Oracle planner: eligibility, view, cost, LPT homes, params_by_home, offsets.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``). Exact Python integers.
"""

from __future__ import annotations


def matrix_view(shape):
    """(rows, cols) view of a tensor shape, or None if it is not eligible.

    owner_planning page, ``select_ge_2d_params``: a tensor takes part iff it
    has at least two dimensions. ``ns_cost_fn``: the tensor is viewed as
    (rows, cols) = (shape[0], product of shape[1:]).

    Pinned by: hand views of 2-D and 3-D shapes in tests/test_oracle_planner.py.
    """
    shape = tuple(int(d) for d in shape)
    if len(shape) < 2:
        return None
    cols = 1
    for d in shape[1:]:
        cols *= d
    return shape[0], cols


def ns_cost(shape, steps: int) -> int:
    """Relative Newton-Schulz work of one tensor.

    owner_planning page, ``ns_cost_fn``: numel * (min(rows, cols) * steps + 1);
    the products cost O(numel * min) per step and the +1 is the linear
    normalisation / elementwise term.

    Pinned by: hand-computed costs (the worked-example tensors and the
    measured shapes) in tests/golden/cost_hand_values.json.
    """
    view = matrix_view(shape)
    if view is None:
        raise ValueError("cost of a tensor with fewer than 2 dims")
    rows, cols = view
    return rows * cols * (min(rows, cols) * steps + 1)


def candidates(split_row, num_homes: int):
    """Eligible owners of one tensor, in buffer order.

    owner_planning page, ``_OwnerWork.candidates`` and ``assign_owner_work``:
    the owner must be a rank holding part of the tensor; candidates are kept
    in buffer order. With no split given, every home is a candidate.
    """
    if split_row is None:
        return list(range(num_homes))
    return [s for s in range(num_homes) if split_row[s] > 0]


def assign_owner_work(costs, cand_lists, num_homes: int):
    """LPT owner assignment.

    owner_planning page, ``assign_owner_work``: tensors with a single candidate
    are assigned first, then the tensors with several candidates in descending
    cost order; each goes to its least-loaded holder, and ties follow buffer
    order. Reading taken where the page is silent: single-candidate tensors go
    in index order, and equal costs keep index order.

    ``costs[i]`` is None for a tensor that does not take part.
    Returns (home, load, order): home[i] is -1 for non-participants, order is
    the assignment order (participants only).

    Pinned by: hand cases (single-candidate-first, ties, descending order),
    the worked example's default balancer, and Graham's LPT bound against an
    exhaustive search on tiny sets (tests/test_oracle_planner.py).
    """
    n = len(costs)
    load = [0] * num_homes
    home = [-1] * n
    order = []

    def place(i):
        best = None
        for s in cand_lists[i]:                  # buffer order
            if best is None or load[s] < load[best]:
                best = s                          # strict '<': first wins ties
        home[i] = best
        load[best] += costs[i]
        order.append(i)

    single = [i for i in range(n) if costs[i] is not None and len(cand_lists[i]) == 1]
    multi = [i for i in range(n) if costs[i] is not None and len(cand_lists[i]) > 1]
    for i in range(n):
        if costs[i] is not None and len(cand_lists[i]) == 0:
            raise ValueError(f"tensor {i} has no candidate home (no rows in any shard)")
    for i in single:
        place(i)
    for i in sorted(multi, key=lambda i: (-costs[i], i)):
        place(i)
    return home, load, order


def plan(shapes, steps: int, num_homes: int, split_rows=None):
    """Select, cost and assign: the whole host-side plan for one set.

    Returns dict(cost, home, load, order); cost[i] is 0 and home[i] is -1 for
    tensors with fewer than 2 dims. split_rows (if given) must list, for each
    tensor, the rows held by each of the num_homes shards, summing to rows.
    """
    n = len(shapes)
    costs, cands = [], []
    for i, shp in enumerate(shapes):
        view = matrix_view(shp)
        if view is None:
            costs.append(None)
            cands.append([])
            continue
        costs.append(ns_cost(shp, steps))
        row = None
        if split_rows is not None:
            row = [int(r) for r in split_rows[i]]
            if len(row) != num_homes or any(r < 0 for r in row):
                raise ValueError(f"bad split for tensor {i}")
            if sum(row) != view[0]:
                raise ValueError(f"split rows of tensor {i} do not sum to {view[0]}")
        cands.append(candidates(row, num_homes))
    home, load, order = assign_owner_work(costs, cands, num_homes)
    return {"cost": [c if c is not None else 0 for c in costs], "home": home,
            "load": load, "order": order}


def params_by_home(num_params: int, home_of, size: int):
    """layer_sharded_a2a page, ``params_by_home``: result[r] lists the params
    homed on r in increasing index order; homes with none get empty lists.

    Pinned by: the worked example (home 0 empty, home 1 = [0, 1]).
    """
    result = [[] for _ in range(size)]
    for i in range(num_params):
        h = home_of[i]
        if not 0 <= h < size:
            raise ValueError(f"home {h} of param {i} out of range")
        result[h].append(i)
    return result


def route_offsets(shapes, split_rows, home, num_shards: int, shard_dim=None):
    """Offsets of every piece in the shard buffers and the home buffers.

    Shard buffer s holds, for every tensor in increasing index order, the rows
    of that tensor it owns (a (rows_s, cols) block, possibly empty), end to
    end -- the per-rank layout of the owner_planning page's worked example
    (rank 0 holds param_0[0:5] then nothing of param_1; rank 1 holds
    param_0[5:6] then all of param_1). Home buffer h holds the complete
    tensors homed on h in increasing index order (layer_sharded_a2a page,
    ``params_by_home`` and ``route_to_ns_home`` returns). A tensor's rows are
    split over shards in buffer order, so shard s holds rows starting at the
    sum of the rows held by the shards before it (``reconstruct_full``
    concatenates per-rank shards in buffer order).

    With ``shard_dim`` (one dimension per tensor; layer_sharded_a2a page,
    ``route_to_ns_home``'s axis-generic ``shard_dim``) the split sizes count
    slices along that dimension instead of rows, and shard s's piece of tensor
    i is that slice: numel / shape[d] * split elements.

    Returns dict with shard_offset[i][s], row_start[i][s], home_offset[i],
    shard_elems[s], home_elems[h] (all in elements).

    Pinned by: the worked example's sizes and offsets (tests/golden) and a
    brute-force element map in tests/test_oracle_route.py.
    """
    n = len(shapes)
    views = [matrix_view(s) for s in shapes]
    if any(v is None for v in views):
        raise ValueError("routed tensors need at least 2 dims")
    shard_offset = [[0] * num_shards for _ in range(n)]
    row_start = [[0] * num_shards for _ in range(n)]
    shard_elems = [0] * num_shards
    home_offset = [0] * n
    home_elems = [0] * num_shards
    for i in range(n):
        d = 0 if shard_dim is None else shard_dim[i]
        shape = tuple(int(x) for x in shapes[i])
        extent = shape[d]
        others = 1
        for k, x in enumerate(shape):
            if k != d:
                others *= x
        if sum(split_rows[i]) != extent:
            raise ValueError(f"split sizes of tensor {i} do not sum to {extent}")
        r0 = 0
        for s in range(num_shards):
            shard_offset[i][s] = shard_elems[s]
            row_start[i][s] = r0
            shard_elems[s] += split_rows[i][s] * others
            r0 += split_rows[i][s]
    groups = params_by_home(n, home, num_shards)
    for h in range(num_shards):
        for i in groups[h]:
            home_offset[i] = home_elems[h]
            rows, cols = views[i]
            home_elems[h] += rows * cols
    return {"shard_offset": shard_offset, "row_start": row_start, "home_offset": home_offset,
            "shard_elems": shard_elems, "home_elems": home_elems}


def wave_plan(shapes, slots: int, ready_order=None):
    """Static partition of the Newton-Schulz work into waves.

    "[GTP][Muon] Optimize Muon step performance" page, "Current Progress",
    the backward/forward overlap item: the NS work is split statically into
    waves sized to the available slots (its example: 3000 tensors on 1000
    slots make 3 waves), and each wave is started as the gradient buckets it
    needs complete. Reading taken where the page is silent: tensors join waves
    in the order their gradients become ready -- ``ready_order``, by default
    reverse index order, the order a backward pass produces them -- and each
    run of ``slots`` consecutive eligible tensors in that order is one wave.
    Tensors with fewer than 2 dims take no part (owner_planning page,
    ``select_ge_2d_params``) and get wave -1.

    Returns (wave_of, num_waves). Pinned by: the page's 3000 / 1000 example,
    hand cases and counting identities in tests/test_oracle_planner.py.
    """
    n = len(shapes)
    if slots < 1:
        raise ValueError("slots must be >= 1")
    order = list(range(n - 1, -1, -1)) if ready_order is None else [int(i) for i in ready_order]
    if sorted(order) != list(range(n)):
        raise ValueError("ready_order is not a permutation")
    wave_of = [-1] * n
    k = 0
    for i in order:
        if matrix_view(shapes[i]) is None:
            continue
        wave_of[i] = k // slots
        k += 1
    return wave_of, (k + slots - 1) // slots
