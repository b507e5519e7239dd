"""Host-side checks of the C ABI (no GPU needed).

* the library loads and exports every function include/ns.h declares;
* ns_plan and the route plan's offsets are bit-exact against the oracle;
* argument errors are reported before anything touches the GPU.
"""

import ctypes
import os
import random
import re

import pytest

import newton_schulz_quintic_amd as nsq
from newton_schulz_quintic_amd import _lib
from oracle import planner
from workloads import dense_transformer, many_small, routed_square_batch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    with open(os.path.join(ROOT, "include", "ns.h")) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ns_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    lib = nsq.lib()
    names = _declared()
    assert "ns_orthogonalize_batched" in names and "ns_pack_shards" in names
    for name in names:
        assert hasattr(lib, name), name
    assert set(names) == set(_lib.EXPORTS)
    assert "gfx950" in nsq.ns_version()


def _compare_plan(shapes, steps, S, split):
    got = nsq.ns_plan(shapes, steps=steps, num_homes=S, split_rows=split)
    want = planner.plan(shapes, steps, S, split)
    assert got["cost"] == want["cost"]
    assert got["home"] == want["home"]
    assert got["load"] == want["load"]
    assert got["order"] == want["order"]
    return got


def test_plan_matches_oracle_hand_and_example():
    _compare_plan([(6, 4), (4, 4)], 5, 2, [[5, 1], [0, 4]])
    _compare_plan([(1, 10), (1, 7), (1, 6), (1, 5)], 1, 2, None)
    _compare_plan([(2, 50), (2, 3)], 1, 2, [[1, 1], [2, 0]])
    _compare_plan([(5,), (2, 3), (7,), (2, 3, 4)], 5, 3, None)


def test_plan_routed_uneven_set():
    ms = routed_square_batch(uneven=True)
    got = _compare_plan(ms.shapes, 5, 4, ms.split_rows)
    # 6 / 5 / 5 / 0 matrices per home; home 3 is empty
    assert [got["home"].count(h) for h in range(4)] == [6, 5, 5, 0]
    ms = routed_square_batch(uneven=False)
    got = _compare_plan(ms.shapes, 5, 4, ms.split_rows)
    assert got["home"] == [0, 1, 2, 3] * 4


@pytest.mark.parametrize("seed", range(25))
def test_plan_random_matches_oracle(seed):
    rng = random.Random(seed)
    S = rng.randint(1, 9)
    n = rng.randint(0, 40)
    shapes = []
    for _ in range(n):
        nd = rng.choice([1, 2, 2, 2, 3])
        shapes.append(tuple(rng.randint(1, 300) for _ in range(nd)))
    split = None
    if rng.random() < 0.6 and n:
        split = []
        for s in shapes:
            rows = s[0]
            cuts = sorted(rng.randint(0, rows) for _ in range(S - 1))
            split.append([b - a for a, b in zip([0] + cuts, cuts + [rows])])
        # tensors of fewer than 2 dims take no part; give them any valid split
    steps = rng.randint(0, 6)
    _compare_plan(shapes, steps, S, split)


def test_plan_large_sets_match_oracle():
    _compare_plan(dense_transformer().shapes, 5, 8, None)
    _compare_plan(many_small().shapes, 5, 8, None)


def _compare_offsets(shapes, split, home, S, elem):
    plan = nsq.ns_route_plan_create(shapes, S, split, home, elem)
    q = nsq.ns_route_plan_query(plan)
    want = planner.route_offsets(shapes, split, home, S)
    assert q["shard_elems"] == want["shard_elems"]
    assert q["home_elems"] == want["home_elems"]
    assert q["home_offset"] == want["home_offset"]
    assert q["shard_offset"] == want["shard_offset"]
    return q


def test_route_offsets_worked_example():
    q = _compare_offsets([(6, 4), (4, 4)], [[5, 1], [0, 4]], [1, 1], 2, 4)
    assert q["home_elems"] == [0, 40] and q["shard_elems"] == [20, 20]


@pytest.mark.parametrize("seed", range(20))
def test_route_offsets_random(seed):
    rng = random.Random(100 + seed)
    S = rng.randint(1, 8)
    n = rng.randint(0, 30)
    shapes, split = [], []
    for _ in range(n):
        nd = rng.randint(2, 4)
        s = tuple([rng.randint(0, 50)] + [rng.randint(0, 7) for _ in range(nd - 1)])
        shapes.append(s)
        cuts = sorted(rng.randint(0, s[0]) for _ in range(S - 1))
        split.append([b - a for a, b in zip([0] + cuts, cuts + [s[0]])])
    home = [rng.randrange(S) for _ in range(n)]
    _compare_offsets(shapes, split, home, S, rng.choice([2, 4]))


def test_route_plan_fingerprint_tracks_inputs():
    a = nsq.ns_route_plan_query(nsq.ns_route_plan_create([(4, 4)], 2, [[2, 2]], [0], 2))
    b = nsq.ns_route_plan_query(nsq.ns_route_plan_create([(4, 4)], 2, [[2, 2]], [0], 2))
    c = nsq.ns_route_plan_query(nsq.ns_route_plan_create([(4, 4)], 2, [[2, 2]], [1], 2))
    d = nsq.ns_route_plan_query(nsq.ns_route_plan_create([(4, 4)], 2, [[1, 3]], [0], 2))
    assert a["fingerprint"] == b["fingerprint"]
    assert len({a["fingerprint"], c["fingerprint"], d["fingerprint"]}) == 3


def _status(fn, *args):
    with pytest.raises(nsq.NSError) as e:
        fn(*args)
    return e.value.name


def test_workspace_size_limits():
    """Byte offsets inside one padded matrix are 32-bit: the largest accepted
    n at m = 256 is the last whose padded X^T (n x (256 + row pad)) stays under
    2^31 bytes; one element more is refused with NS_ERR_OVERFLOW, wide or tall."""
    for dtype, es, n_max in ((nsq.NS_BF16, 2, 2796032), (nsq.NS_F32, 4, 1677568)):
        assert n_max * (256 + 256 // es) * es < 2 ** 31 <= (n_max + 256) * (256 + 256 // es) * es
        for shape in ((256, n_max), (n_max, 256)):
            nsq.ns_workspace_bytes([shape], dtype)
        for shape in ((256, n_max + 1), (n_max + 1, 256)):
            assert _status(nsq.ns_workspace_bytes, [shape], dtype) == "NS_ERR_OVERFLOW"


def test_plan_errors():
    assert _status(nsq.ns_plan, [(4, 5)], 5, 2, [[1, 2]]) == "NS_ERR_SPLIT_SUM"
    assert _status(nsq.ns_plan, [(0, 5)], 5, 2, [[0, 0]]) == "NS_ERR_NO_CANDIDATE"
    assert _status(nsq.ns_plan, [(4, 5)], 5, 2, [[-1, 5]]) == "NS_ERR_INVALID_ARG"
    assert _status(nsq.ns_plan, [(4, 5)], -1, 2) == "NS_ERR_INVALID_ARG"
    assert _status(nsq.ns_plan, [(4, 5)], 5, 0) == "NS_ERR_INVALID_ARG"
    assert _status(nsq.ns_plan, [(4, 5)], 5, 65) == "NS_ERR_INVALID_ARG"
    assert _status(nsq.ns_plan, [(2 ** 31, 2 ** 31)], 5, 1) == "NS_ERR_OVERFLOW"
    assert _status(nsq.ns_plan, [(2 ** 40, 2 ** 40)], 5, 1) == "NS_ERR_OVERFLOW"
    assert "overflow" in nsq.ns_last_error()
    lib = nsq.lib()
    assert lib.ns_plan(1, None, 5, 1, None, None, None, None, None) == -1
    assert lib.ns_plan(-1, None, 5, 1, None, None, None, None, None) == -1
    assert lib.ns_plan(0, None, 5, 1, None, None, None, None, None) == 0


def test_route_plan_errors():
    assert _status(nsq.ns_route_plan_create, [(4, 4)], 2, [[2, 2]], [2], 2) == "NS_ERR_HOME_RANGE"
    assert _status(nsq.ns_route_plan_create, [(4, 4)], 2, [[2, 2]], [-1], 2) == "NS_ERR_HOME_RANGE"
    assert _status(nsq.ns_route_plan_create, [(4, 4)], 2, [[2, 1]], [0], 2) == "NS_ERR_SPLIT_SUM"
    assert _status(nsq.ns_route_plan_create, [(4, 4)], 2, [[2, 2]], [0], 3) == "NS_ERR_DTYPE"
    assert _status(nsq.ns_route_plan_create, [(4,)], 1, [[4]], [0], 2) == "NS_ERR_INVALID_ARG"
    assert _status(nsq.ns_route_plan_create, [(4, 4)], 0, [], [0], 2) == "NS_ERR_INVALID_ARG"
    big = 2 ** 62
    assert _status(nsq.ns_route_plan_create, [(big, 2)], 1, [[big]], [0], 2) == "NS_ERR_OVERFLOW"
    lib = nsq.lib()
    out = ctypes.c_void_p()
    assert lib.ns_route_plan_create(1, None, 1, None, None, 2, ctypes.byref(out)) == -1
    assert lib.ns_route_plan_create(0, None, 1, None, None, 2, None) == -1
    # an empty plan is fine
    p = nsq.ns_route_plan_create([], 3, [], [], 2)
    assert nsq.ns_route_plan_query(p)["shard_elems"] == [0, 0, 0]
    # pack before upload: plan mismatch (checked on the host, nothing launched)
    p = nsq.ns_route_plan_create([(4, 4)], 1, [[4]], [0], 2)
    assert lib.ns_pack_shards(p.handle, None, None, None) in (-1, -6)
    assert lib.ns_pack_shards(None, None, None, None) == -1


def test_workspace_and_batched_errors():
    b, mb = nsq.ns_workspace_bytes([(1024, 1024)] * 3 + [(5,)], nsq.NS_BF16)
    assert b > mb > 0
    one, _ = nsq.ns_workspace_bytes([(1024, 1024)], nsq.NS_BF16)
    assert b > 2 * (one - 4096)
    # X ping/pong, A and B', rows padded by 256 bytes, plus tables (no X^T)
    arrays = 4 * 1024 * (1024 * 2 + 256)
    assert arrays <= one < arrays + (1 << 20)
    # f32 needs about twice the buffers
    b32, _ = nsq.ns_workspace_bytes([(1024, 1024)], nsq.NS_F32)
    assert b32 > 1.8 * one       # fixed 256-byte row pad is not doubled
    assert _status(nsq.ns_workspace_bytes, [(4, 4)], 7) == "NS_ERR_DTYPE"
    lib = nsq.lib()
    # n == 0 is a no-op; these all fail in host validation, before any HIP call
    assert lib.ns_orthogonalize_batched(0, None, None, None, 0, 5, 1.0, 0.0, 0.0, 1e-7, None, None, 0,
                                        None) == 0
    sh = _lib._shapes([(4, 4)])
    ptrs = _lib._arr(ctypes.c_void_p, [256])
    args = lambda dtype=0, steps=5, eps=1e-7, order=None, ws=None, wsb=0: (  # noqa: E731
        1, ctypes.addressof(sh), ctypes.addressof(ptrs), ctypes.addressof(ptrs), dtype, steps, 3.4, -4.7,
        2.0, eps, order, ws, wsb, None)
    assert lib.ns_orthogonalize_batched(*args(dtype=5)) == -8
    assert lib.ns_orthogonalize_batched(*args(steps=-1)) == -1
    assert lib.ns_orthogonalize_batched(*args(eps=-1.0)) == -1
    bad_order = _lib._arr(ctypes.c_int32, [3])
    assert lib.ns_orthogonalize_batched(*args(order=ctypes.addressof(bad_order))) == -1
    assert lib.ns_orthogonalize_batched(*args()) == -7          # no workspace
    assert lib.ns_orthogonalize_batched(*args(ws=4096, wsb=16)) == -7   # too small
    assert lib.ns_orthogonalize_batched(*args(ws=4100, wsb=1 << 30)) == -7  # misaligned
    odd = _lib._arr(ctypes.c_void_p, [257])
    assert lib.ns_orthogonalize_batched(1, ctypes.addressof(sh), ctypes.addressof(odd),
                                        ctypes.addressof(odd), 0, 5, 3.4, -4.7, 2.0, 1e-7, None, 4096,
                                        1 << 30, None) == -1
    assert "aligned" in nsq.ns_last_error()


def test_routed_workspace_and_errors():
    ms = routed_square_batch(uneven=True)
    plan = nsq.ns_route_plan_create(ms.shapes, 4, ms.split_rows, [0] * ms.n, 2)
    b, mb = nsq.ns_routed_workspace_bytes(plan, nsq.NS_BF16)
    ub, umb = nsq.ns_workspace_bytes(ms.shapes, nsq.NS_BF16)
    # the same buffers; only the piece table grows (one piece per nonzero split)
    assert 0 <= b - ub <= 4096 and 0 <= mb - umb <= 4096
    assert _status(nsq.ns_routed_workspace_bytes, plan, nsq.NS_F32) == "NS_ERR_PLAN_MISMATCH"
    assert _status(nsq.ns_routed_workspace_bytes, plan, 9) == "NS_ERR_DTYPE"
    lib = nsq.lib()
    bs = _lib._SZ(0)
    assert lib.ns_routed_workspace_bytes(None, 0, ctypes.addressof(bs), None) == -1
    # host validation only: nothing is launched
    nul = _lib._arr(ctypes.c_void_p, [None] * 4)
    ok = _lib._arr(ctypes.c_void_p, [256] * 4)
    call = lambda p, i, o, dtype=0, steps=5, eps=1e-7: lib.ns_orthogonalize_routed(  # noqa: E731
        p, i, o, dtype, steps, 3.4, -4.7, 2.0, eps, None, None, 0, None)
    assert call(None, ctypes.addressof(ok), ctypes.addressof(ok)) == -1
    assert call(plan.handle, ctypes.addressof(ok), ctypes.addressof(ok), dtype=1) == -6
    assert call(plan.handle, ctypes.addressof(ok), ctypes.addressof(ok), steps=-1) == -1
    assert call(plan.handle, ctypes.addressof(nul), ctypes.addressof(ok)) == -1
    assert call(plan.handle, None, ctypes.addressof(ok)) == -1
    odd = _lib._arr(ctypes.c_void_p, [257] * 4)
    assert call(plan.handle, ctypes.addressof(odd), ctypes.addressof(ok)) == -1
    assert call(plan.handle, ctypes.addressof(ok), ctypes.addressof(ok)) == -7   # no workspace
    empty = nsq.ns_route_plan_create([], 2, [], [], 2)
    assert call(empty.handle, None, None) == 0


@pytest.mark.parametrize("seed", range(12))
def test_wave_plan_matches_oracle(seed):
    rng = random.Random(700 + seed)
    n = rng.randint(0, 50)
    shapes = [tuple(rng.randint(0, 9) for _ in range(rng.choice([1, 2, 3]))) for _ in range(n)]
    slots = rng.randint(1, 10)
    order = None
    if rng.random() < 0.5:
        order = list(range(n))
        rng.shuffle(order)
    assert nsq.ns_wave_plan(shapes, slots, order) == tuple(planner.wave_plan(shapes, slots, order))


def test_wave_plan_and_waves_errors():
    assert nsq.ns_wave_plan([(8, 8)] * 3000, 1000)[1] == 3
    assert _status(nsq.ns_wave_plan, [(2, 2)], 0) == "NS_ERR_INVALID_ARG"
    assert _status(nsq.ns_wave_plan, [(2, 2), (3, 3)], 1, [0, 0]) == "NS_ERR_INVALID_ARG"
    assert _status(nsq.ns_wave_plan, [(2, 2)], 1, [1]) == "NS_ERR_INVALID_ARG"
    lib = nsq.lib()
    sh = _lib._shapes([(4, 4)])
    ptrs = _lib._arr(ctypes.c_void_p, [256])
    w = _lib._arr(ctypes.c_int32, [1])
    call = lambda waves, num: lib.ns_orthogonalize_waves(  # noqa: E731
        1, ctypes.addressof(sh), ctypes.addressof(ptrs), ctypes.addressof(ptrs), 0, 5, 3.4, -4.7, 2.0, 1e-7,
        waves, num, None, None, 0, None)
    assert call(ctypes.addressof(w), 1) == -1          # wave 1 >= num_waves 1
    assert call(None, 1) == -1
    assert call(ctypes.addressof(w), -1) == -1
    assert call(ctypes.addressof(w), 2) == -7          # no workspace


def test_strided_errors():
    lib = nsq.lib()
    sh = _lib._shapes([(4, 6)])
    ptrs = _lib._arr(ctypes.c_void_p, [256])
    call = lambda li, lo: lib.ns_orthogonalize_strided(  # noqa: E731
        1, ctypes.addressof(sh), ctypes.addressof(ptrs), li, ctypes.addressof(ptrs), lo, 0, 5, 3.4, -4.7, 2.0,
        1e-7, None, None, 0, None)
    short = _lib._arr(ctypes.c_int64, [5])
    ok = _lib._arr(ctypes.c_int64, [8])
    assert call(ctypes.addressof(short), None) == -1      # row stride below the row length
    assert call(None, ctypes.addressof(short)) == -1
    huge = _lib._arr(ctypes.c_int64, [2 ** 62])
    assert call(ctypes.addressof(huge), None) == -5
    assert call(ctypes.addressof(ok), ctypes.addressof(ok)) == -7   # valid; no workspace
    assert call(None, None) == -7


@pytest.mark.parametrize("seed", range(15))
def test_route_offsets_axis_random(seed):
    rng = random.Random(300 + seed)
    S = rng.randint(1, 6)
    n = rng.randint(0, 20)
    shapes, split, dims = [], [], []
    for _ in range(n):
        nd = rng.randint(2, 4)
        s = tuple(rng.randint(0, 9) for _ in range(nd))
        d = rng.randrange(nd)
        cuts = sorted(rng.randint(0, s[d]) for _ in range(S - 1))
        split.append([b - a for a, b in zip([0] + cuts, cuts + [s[d]])])
        shapes.append(s)
        dims.append(d)
    home = [rng.randrange(S) for _ in range(n)]
    elem = rng.choice([2, 4])
    q = nsq.ns_route_plan_query(nsq.ns_route_plan_create_axis(shapes, S, split, dims, home, elem))
    want = planner.route_offsets(shapes, split, home, S, shard_dim=dims)
    for key in ("shard_elems", "home_elems", "home_offset", "shard_offset"):
        assert q[key] == want[key], key


def test_route_plan_axis_errors():
    assert _status(nsq.ns_route_plan_create_axis, [(4, 6)], 2, [[3, 3]], [2], [0], 2) == "NS_ERR_INVALID_ARG"
    assert _status(nsq.ns_route_plan_create_axis, [(4, 6)], 2, [[3, 2]], [1], [0], 2) == "NS_ERR_SPLIT_SUM"
    # dim 0 through the axis entry point equals the row plan, fingerprint included
    a = nsq.ns_route_plan_query(nsq.ns_route_plan_create([(4, 6)], 2, [[1, 3]], [1], 2))
    b = nsq.ns_route_plan_query(nsq.ns_route_plan_create_axis([(4, 6)], 2, [[1, 3]], [0], [1], 2))
    assert a == b
    c = nsq.ns_route_plan_query(nsq.ns_route_plan_create_axis([(4, 6)], 2, [[3, 3]], [1], [1], 2))
    assert c["fingerprint"] != a["fingerprint"]
    # fused routing refuses a tensor split along dim 1 over several shards
    plan = nsq.ns_route_plan_create_axis([(4, 6)], 2, [[3, 3]], [1], [0], 2)
    assert _status(nsq.ns_routed_workspace_bytes, plan, nsq.NS_BF16) == "NS_ERR_PLAN_MISMATCH"
    whole = nsq.ns_route_plan_create_axis([(4, 6)], 2, [[0, 6]], [1], [0], 2)
    assert nsq.ns_routed_workspace_bytes(whole, nsq.NS_BF16)[0] > 0


def test_gram_workspace_and_errors():
    b, mb = nsq.ns_gram_workspace_bytes([(1024, 4096)] * 2, nsq.NS_BF16)
    # fp32: X0 (1024 x 4096) + nine 1024 x 1024 arrays, rows padded by 256 bytes
    one = 1024 * (4096 * 4 + 256) + 9 * 1024 * (1024 * 4 + 256)
    assert mb >= one and b >= 2 * one
    assert mb < one + (1 << 20)      # plus tables only
    assert b == nsq.ns_gram_workspace_bytes([(1024, 4096)] * 2, nsq.NS_F32)[0]
    lib = nsq.lib()
    sh = _lib._shapes([(4, 4)])
    ptrs = _lib._arr(ctypes.c_void_p, [256])
    call = lambda ridge, steps=5: lib.ns_orthogonalize_gram(  # noqa: E731
        1, ctypes.addressof(sh), ctypes.addressof(ptrs), ctypes.addressof(ptrs), 0, steps, 3.4, -4.7, 2.0, 1e-7,
        ridge, None, None, 0, None)
    assert call(-1.0) == -1
    assert call(float("inf")) == -1
    assert call(0.0, steps=-2) == -1
    assert call(1e-3) == -7      # valid; no workspace


def test_route_plan_bands_strided_pieces():
    # a piece sliced along a later dimension is moved in bands of about
    # 256 KiB of home rows (one 64-byte table entry per band and shard); row
    # pieces and small strided ones stay whole
    entry = 64
    rows = nsq.ns_route_plan_query(nsq.ns_route_plan_create_axis([(4096, 4096)], 4, [[1024] * 4], [0], [0], 2))
    assert rows["device_table_bytes"] == 4 * entry
    # 4096 home rows of 8 KiB: bands of 32 rows, 128 bands x 4 shards
    cols = nsq.ns_route_plan_query(nsq.ns_route_plan_create_axis([(4096, 4096)], 4, [[1024] * 4], [1], [0], 2))
    assert cols["device_table_bytes"] == 128 * 4 * entry
    # 1000 home rows of 8200 bytes: bands of 31 rows, the last one ragged (33 bands), one zero-width shard
    rag = nsq.ns_route_plan_query(nsq.ns_route_plan_create_axis([(1000, 4100)], 4, [[1025, 0, 2050, 1025]], [1], [0],
                                                                2))
    assert rag["device_table_bytes"] == 33 * 3 * entry
    small = nsq.ns_route_plan_query(nsq.ns_route_plan_create_axis([(30, 64)], 2, [[32, 32]], [1], [0], 2))
    assert small["device_table_bytes"] == max(16, 2 * entry)


def test_errors_come_before_any_enqueue():
    # Every argument error is found before the first HIP call: without a GPU
    # any HIP call fails with NS_ERR_HIP (-9), so each of these returning its
    # own code shows that nothing was enqueued first. The event handle is a
    # stand-in that must never be touched.
    lib = nsq.lib()
    shapes = [(300, 200), (64, 1000), (5, 7)]
    sh = _lib._shapes(shapes)
    need, minimum = nsq.ns_workspace_bytes(shapes, nsq.NS_BF16)
    assert minimum < need
    ptrs = _lib._arr(ctypes.c_void_p, [4096, 8192, 16384])
    wave = _lib._arr(ctypes.c_int32, [0, 1, 1])
    events = _lib._arr(ctypes.c_void_p, [0x1000, 0x2000])

    def waves(ws, nbytes):
        return lib.ns_orthogonalize_waves(3, ctypes.addressof(sh), ctypes.addressof(ptrs), ctypes.addressof(ptrs),
                                          0, 5, 3.4, -4.7, 2.0, 1e-7, ctypes.addressof(wave), 2,
                                          ctypes.addressof(events), ws, nbytes, None)
    assert waves((1 << 20) + 128, need) == -7       # misaligned workspace: no event wait enqueued
    assert waves(1 << 20, minimum - 1) == -7        # below the minimum
    assert waves(None, need) == -7

    def batched(ws, nbytes, order=None):
        return lib.ns_orthogonalize_batched(3, ctypes.addressof(sh), ctypes.addressof(ptrs), ctypes.addressof(ptrs),
                                            0, 5, 3.4, -4.7, 2.0, 1e-7, order, ws, nbytes, None)
    # a minimum workspace makes several groups; every one is planned first
    bad = _lib._arr(ctypes.c_int32, [0, 0, 1])
    assert batched(1 << 20, minimum, ctypes.addressof(bad)) == -1
    assert batched((1 << 20) + 128, minimum) == -7
    assert batched(1 << 20, minimum - 1) == -7


def test_noalloc_errors_before_any_hip_call():
    # Without a GPU every HIP call fails (NS_ERR_HIP); these return their own
    # codes first: bad dtype, and a tensor larger than the 64 MiB scratch.
    lib = nsq.lib()
    sh = _lib._shapes([(4096, 4096)])
    ptrs = _lib._arr(ctypes.c_void_p, [4096])
    call = lambda dtype: lib.ns_orthogonalize_batched_noalloc(  # noqa: E731
        1, ctypes.addressof(sh), ctypes.addressof(ptrs), ctypes.addressof(ptrs), dtype, 5, 3.4, -4.7, 2.0, 1e-7,
        None, None)
    assert call(7) == -8
    assert call(0) == -7
    assert "64 MiB" in nsq.ns_last_error() or "scratch" in nsq.ns_last_error()
    assert lib.ns_orthogonalize_batched_noalloc(0, None, None, None, 0, 5, 3.4, -4.7, 2.0, 1e-7, None, None) == 0
