"""GPU parity of pack / unpack for shards cut along any dimension: bit-exact.

Cases: random tensors (2-4 dims) split along a random dimension with zero
widths, in 2- and 4-byte elements, at sizes whose strided runs span several
16 KiB chunks and odd widths that force 4- and 2-byte units; 4096-wide
column shards (the TP stage's partition_dim = 1); and the two-stage exchange
(rows within each column group, then columns) rebuilding the full tensor.
"""

import numpy as np
import pytest

import newton_schulz_quintic_amd as nsq
from oracle import route
from tests.helpers import log

pytestmark = pytest.mark.gpu


def _dev(x):
    import torch
    return torch.from_numpy(x.view(np.int16) if x.dtype == np.uint16 else x.view(np.int32)).cuda() \
        if x.size else None


def _host(t, dtype):
    return t.cpu().numpy().view(dtype)


def _case(rng, S, shapes, dims, elem):
    dtype = np.uint16 if elem == 2 else np.uint32
    split, fulls = [], []
    for shape, d in zip(shapes, dims):
        cuts = np.sort(rng.integers(0, shape[d] + 1, size=S - 1))
        split.append(np.diff(np.concatenate([[0], cuts, [shape[d]]])).astype(int).tolist())
        fulls.append(rng.integers(0, 2 ** (8 * elem) - 1, size=shape, dtype=dtype))
    shards = [[] for _ in range(S)]
    for f, sp, d in zip(fulls, split, dims):
        for s, blk in enumerate(np.split(f, np.cumsum(sp)[:-1], axis=d)):
            shards[s].append(blk.ravel())
    shards = [np.concatenate(p) if p else np.zeros(0, dtype) for p in shards]
    return split, shards, dtype


def _roundtrip(shapes, split, dims, home, S, shards_host, elem, dtype):
    import torch
    plan = nsq.ns_route_plan_create_axis(shapes, S, split, dims, home, elem)
    q = nsq.ns_route_plan_query(plan)
    nsq.ns_route_plan_upload(plan)
    tdt = torch.int16 if elem == 2 else torch.int32
    shards = [_dev(x) for x in shards_host]
    homes = [torch.full((n,), -1, dtype=tdt, device="cuda") if n else None for n in q["home_elems"]]
    nsq.ns_pack_shards(plan, shards, homes)
    torch.cuda.synchronize()
    want = route.pack_axis(shards_host, shapes, split, dims, home, S)
    for h in range(S):
        got = _host(homes[h], dtype) if homes[h] is not None else np.zeros(0, dtype)
        assert np.array_equal(got, want[h]), f"home {h}"
    back = [torch.full((n,), -1, dtype=tdt, device="cuda") if n else None for n in q["shard_elems"]]
    nsq.ns_unpack_shards(plan, homes, back)
    torch.cuda.synchronize()
    for s in range(S):
        if q["shard_elems"][s]:
            assert np.array_equal(_host(back[s], dtype), shards_host[s]), f"shard {s}"
    return homes


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("elem", [2, 4])
def test_random_axes(seed, elem):
    rng = np.random.default_rng(1000 + seed)
    S = int(rng.integers(1, 6))
    n = int(rng.integers(1, 9))
    shapes, dims = [], []
    for _ in range(n):
        nd = int(rng.integers(2, 5))
        # large enough that runs cross chunk boundaries; odd extents for narrow units
        base = [int(rng.integers(1, 40)) for _ in range(nd)]
        base[-1] = int(rng.choice([1, 3, 8, 64, 257, 1024]))
        shapes.append(tuple(base))
        dims.append(int(rng.integers(0, nd)))
    split, shards, dtype = _case(rng, S, shapes, dims, elem)
    home = [int(rng.integers(0, S)) for _ in range(n)]
    log(f"route axis: seed {seed} elem {elem} S {S} shapes {shapes} dims {dims}")
    _roundtrip(shapes, split, dims, home, S, shards, elem, dtype)


def test_column_shards_wide():
    rng = np.random.default_rng(7)
    shapes = [(4096, 4096), (1024, 4096), (4096, 1024), (512, 14336)]
    dims = [1, 1, 1, 1]
    S = 4
    split, shards, dtype = _case(rng, S, shapes, dims, 2)
    log("route axis: 4-way column shards, transformer shapes")
    _roundtrip(shapes, split, dims, [0, 1, 2, 3], S, shards, 2, dtype)


def test_two_stage_rows_then_columns():
    import torch
    rng = np.random.default_rng(8)
    P, Q, R, C = 1000, 777, 3, 4
    full = rng.integers(0, 65535, size=(P, Q), dtype=np.uint16)
    rsplit = [300, 0, 700]
    csplit = [200, 177, 0, 400]
    rows = np.split(full, np.cumsum(rsplit)[:-1], axis=0)
    col_idx = np.split(np.arange(Q), np.cumsum(csplit)[:-1])
    log("route axis: two-stage exchange (rows, then columns)")
    stage1 = []
    for t in range(C):
        w = len(col_idx[t])
        shards_host = [np.ascontiguousarray(rows[r][:, col_idx[t]]).ravel() for r in range(R)]
        homes = _roundtrip([(P, w)], [rsplit], [0], [0], R, shards_host, 2, np.uint16)
        stage1.append(_host(homes[0], np.uint16) if homes[0] is not None else np.zeros(0, np.uint16))
    homes = _roundtrip([(P, Q)], [csplit], [1], [2], C, stage1, 2, np.uint16)
    assert np.array_equal(_host(homes[2], np.uint16).reshape(P, Q), full)
    assert torch.cuda.is_available()


@pytest.mark.parametrize("max_grid", ["1", "5"])
def test_axes_several_chunks_per_workgroup(monkeypatch, max_grid):
    # workgroups walking several chunks across strided pieces
    monkeypatch.setenv("NS_ROUTE_MAX_GRID", max_grid)
    for seed in range(3):
        test_random_axes(seed, 2)
    test_random_axes(3, 4)
    test_column_shards_wide()


@pytest.mark.parametrize("elem", [2, 4])
def test_banded_strided_pieces_ragged(elem):
    # strided pieces are moved in bands of home rows (about 256 KiB of rows per
    # band): row counts that are not a multiple of the band, odd widths (narrow
    # units), a 3-dimensional tensor cut along its last dimension
    rng = np.random.default_rng(13 + elem)
    shapes = [(1000, 4100), (64, 300, 1000), (2047, 2048)]
    dims = [1, 2, 1]
    S = 4
    split, shards, dtype = _case(rng, S, shapes, dims, elem)
    log(f"route axis: banded strided pieces, elem {elem}, splits {split}")
    _roundtrip(shapes, split, dims, [1, 0, 3], S, shards, elem, dtype)
