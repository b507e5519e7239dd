"""GPU parity of pack / unpack against the oracle: bit-exact.

Pack gathers every tensor's row pieces from the S shard buffers into its home
buffer; unpack scatters them back. Cases: the owner_planning page's worked
example, the 16 x 1024^2 set in 4 even and 4 uneven shards (one home empty),
random uneven splits with zero-row pieces and odd column counts (unaligned
pieces), a single shard, and 4-byte elements.
"""

import numpy as np
import pytest

import newton_schulz_quintic_amd as nsq
from oracle import route
from tests.helpers import log, to_device, to_host
from workloads import host_matrix, routed_square_batch

pytestmark = pytest.mark.gpu


def _shards_from_fulls(fulls, split_rows, S):
    parts = [[] for _ in range(S)]
    for f, split in zip(fulls, split_rows):
        for s, blk in enumerate(np.split(f.reshape(f.shape[0], -1), np.cumsum(split)[:-1], axis=0)):
            parts[s].append(blk.ravel())
    return [np.concatenate(p) for p in parts]


def _run(shapes, split_rows, home, S, shards_host, dtype):
    torch = pytest.importorskip("torch")
    elem = 2 if dtype == "bf16" else 4
    plan = nsq.ns_route_plan_create(shapes, S, split_rows, home, elem)
    q = nsq.ns_route_plan_query(plan)
    nsq.ns_route_plan_upload(plan)
    shards = [to_device(x, dtype) if x.size else None for x in shards_host]
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    homes = [torch.full((n,), float("nan"), dtype=tdt, device="cuda") if n else None
             for n in q["home_elems"]]
    nsq.ns_pack_shards(plan, shards, homes)
    torch.cuda.synchronize()
    got = [to_host(h, dtype) if h is not None else np.zeros(0, shards_host[0].dtype) for h in homes]
    want = route.pack(shards_host, shapes, split_rows, home, S)
    for h in range(S):
        assert got[h].shape == want[h].shape
        assert np.array_equal(got[h].view(np.uint8), want[h].view(np.uint8)), f"home {h}"
    back = [torch.full((n,), float("nan"), dtype=tdt, device="cuda") if n else None
            for n in q["shard_elems"]]
    nsq.ns_unpack_shards(plan, homes, back)
    torch.cuda.synchronize()
    for s in range(S):
        if q["shard_elems"][s]:
            assert np.array_equal(to_host(back[s], dtype).view(np.uint8), shards_host[s].view(np.uint8))
    return got


def test_worked_example_fp32():
    log("route: owner_planning worked example")
    flat = np.arange(40, dtype=np.float32)
    got = _run([(6, 4), (4, 4)], [[5, 1], [0, 4]], [1, 1], 2, [flat[:20], flat[20:]], "f32")
    assert got[0].size == 0
    assert np.array_equal(got[1], np.concatenate([flat[0:20], flat[20:24], flat[24:40]]))


@pytest.mark.parametrize("uneven", [False, True])
def test_square_set_four_shards(uneven):
    ms = routed_square_batch(uneven)
    log(f"route: {ms.name}")
    fulls = [host_matrix(ms.seed, i, s) for i, s in enumerate(ms.shapes)]
    shards = _shards_from_fulls(fulls, ms.split_rows, 4)
    home = nsq.ns_plan(ms.shapes, 5, 4, ms.split_rows)["home"]
    got = _run(ms.shapes, ms.split_rows, home, 4, shards, "bf16")
    if uneven:
        assert got[3].size == 0
    # each home holds its matrices, complete, in index order
    for h in range(4):
        mine = [fulls[i].ravel() for i in range(16) if home[i] == h]
        if mine:
            assert np.array_equal(got[h], np.concatenate(mine))


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_random_uneven_with_zeros(seed, dtype):
    rng = np.random.default_rng(500 + seed)
    S = int(rng.integers(1, 9))
    n = int(rng.integers(1, 14))
    shapes, fulls, split = [], [], []
    for i in range(n):
        rows = int(rng.integers(0, 700))
        cols = int(rng.integers(1, 300)) | 1         # odd widths: pieces start unaligned
        shapes.append((rows, cols))
        fulls.append(host_matrix(seed, i, (rows, cols), dtype=dtype))
        cuts = np.sort(rng.integers(0, rows + 1, size=S - 1))
        split.append(np.diff(np.concatenate([[0], cuts, [rows]])).astype(int).tolist())
    home = [int(rng.integers(0, S)) for _ in range(n)]
    log(f"route: random seed={seed} dtype={dtype} S={S} n={n}")
    shards = _shards_from_fulls(fulls, split, S)
    _run(shapes, split, home, S, shards, dtype)


def test_single_shard_and_large_pieces():
    rng = np.random.default_rng(9)
    shapes = [(3000, 4096), (17, 33), (1024, 1024)]
    fulls = [rng.integers(0, 65535, size=s, dtype=np.uint16) for s in shapes]
    log("route: single shard")
    _run(shapes, [[s[0]] for s in shapes], [0, 0, 0], 1, [np.concatenate([f.ravel() for f in fulls])],
         "bf16")


@pytest.mark.parametrize("cols,tail", [(4096, (512, 1024)), (4097, (1000, 333))])
def test_plan_beyond_last_level_cache(cols, tail):
    # about 302 MB moved per launch, more than the 256 MB last-level cache: the
    # kernel that loads and stores with non-temporal hints; 16-byte aligned
    # pieces (4096 columns), then pieces at 2-byte offsets (odd column counts)
    rng = np.random.default_rng(12)
    shapes = [(4096, cols)] * 9 + [tail]
    split = [[1024, 1100, 972, 1000]] * 9 + [[tail[0] // 4, 0, tail[0] // 2, tail[0] - 3 * (tail[0] // 4)]]
    home = [0, 1, 2, 3, 0, 1, 2, 3, 0, 1]
    fulls = [rng.integers(0, 65535, size=s, dtype=np.uint16) for s in shapes]
    assert sum(s[0] * s[1] for s in shapes) * 2 > 256 << 20
    log(f"route: beyond the last-level cache, cols={cols}")
    _run(shapes, split, home, 4, _shards_from_fulls(fulls, split, 4), "bf16")


@pytest.mark.parametrize("max_grid", ["1", "3", "7"])
def test_several_chunks_per_workgroup(monkeypatch, max_grid):
    # plans under 128 GiB give each workgroup one 16 KiB chunk; a lowered cap
    # makes workgroups walk several chunks and cross piece boundaries
    monkeypatch.setenv("NS_ROUTE_MAX_GRID", max_grid)
    log(f"route: NS_ROUTE_MAX_GRID={max_grid}")
    test_square_set_four_shards(True)
    for seed in range(3):
        test_random_uneven_with_zeros(seed, "bf16")
    test_random_uneven_with_zeros(3, "f32")
