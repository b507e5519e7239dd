"""GPU parity of ns_orthogonalize_routed (Newton-Schulz read from and written
back to the shard buffers, no home buffers).

Bar: bit-identical to ns_pack_shards -> ns_orthogonalize_batched ->
ns_unpack_shards on the same plan (and so to the unrouted batched call on the
full tensors), and within the fp64 oracle's tolerance. Cases: the 16 x 1024^2
set in 4 uneven shards with an empty home; ragged wide / tall / 3-D tensors
with zero-row pieces and odd column counts (unaligned pieces); a tall tensor
cut into 1-3 row pieces over 64 shards (many pieces per tile); in place; fp32;
zero steps; a workspace that holds one tensor at a time.
"""

import random

import numpy as np
import pytest

import newton_schulz_quintic_amd as nsq
from tests.helpers import TOL, log, oracle_ns, to_device, to_host
from workloads import DEFAULT_EPS, QUINTIC, host_matrix, routed_square_batch

pytestmark = pytest.mark.gpu


def _split(full, split):
    cols = int(np.prod(full.shape[1:]))
    return np.split(full.reshape(full.shape[0], cols), np.cumsum(split)[:-1], axis=0)


def _shards(fulls, split_rows, S, dtype):
    zero = np.uint16 if dtype == "bf16" else np.float32
    parts = [[np.zeros(0, zero)] for _ in range(S)]
    for f, split in zip(fulls, split_rows):
        for s, blk in enumerate(_split(f, split)):
            parts[s].append(blk.ravel())
    return [np.concatenate(p) for p in parts]


def _dev(x, dtype):
    return to_device(x, dtype) if x.size else None


def _fused(plan, shards_host, dtype, steps=5, workspace=None, in_place=False):
    import torch
    code = nsq.NS_BF16 if dtype == "bf16" else nsq.NS_F32
    ins = [_dev(x, dtype) for x in shards_host]
    outs = ins if in_place else [None if x is None else torch.full_like(x, float("nan")) for x in ins]
    nsq.ns_orthogonalize_routed(plan, ins, outs, code, steps=steps, coeffs=QUINTIC, eps=DEFAULT_EPS,
                                workspace=workspace)
    torch.cuda.synchronize()
    return [to_host(o, dtype) if o is not None else np.zeros(0, x.dtype) for o, x in zip(outs, shards_host)]


def _unfused(plan, shapes, shards_host, dtype, steps=5):
    """pack -> batched NS on the home buffers -> unpack."""
    import torch
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    q = nsq.ns_route_plan_query(plan)
    nsq.ns_route_plan_upload(plan)
    shards = [_dev(x, dtype) for x in shards_host]
    homes = [torch.empty(n, dtype=tdt, device="cuda") if n else None for n in q["home_elems"]]
    nsq.ns_pack_shards(plan, shards, homes)
    home_of = plan.home
    views = []
    for i, s in enumerate(shapes):
        numel = int(np.prod(s))
        if numel == 0:
            continue
        off = q["home_offset"][i]
        views.append(homes[home_of[i]][off:off + numel].view(s))
    res = [torch.empty_like(v) for v in views]
    nsq.ns_orthogonalize_batched(views, res, steps=steps, coeffs=QUINTIC, eps=DEFAULT_EPS)
    for v, r in zip(views, res):
        v.copy_(r)
    nsq.ns_unpack_shards(plan, homes, shards)
    torch.cuda.synchronize()
    return [to_host(x, dtype) if x is not None else np.zeros(0, h.dtype) for x, h in zip(shards, shards_host)]


def _plan(shapes, split_rows, S, dtype, home=None):
    if home is None:
        home = nsq.ns_plan(shapes, 5, S, split_rows)["home"]
    plan = nsq.ns_route_plan_create(shapes, S, split_rows, home, 2 if dtype == "bf16" else 4)
    plan.home = home
    return plan


def _oracle_check(fulls, split_rows, S, out_shards, dtype, steps=5, check=None):
    """Each tensor's rows, gathered from the output shards, against the oracle."""
    q_off = [0] * S
    for i, (f, split) in enumerate(zip(fulls, split_rows)):
        cols = int(np.prod(f.shape[1:])) if f.ndim > 1 else 1
        rows = []
        for s, r in enumerate(split):
            rows.append(out_shards[s][q_off[s]:q_off[s] + r * cols].reshape(r, cols))
            q_off[s] += r * cols
        if check is not None and i not in check:
            continue
        if f.size == 0:
            continue
        got = np.concatenate(rows, axis=0)
        got = (got.astype(np.uint32) << 16).view(np.float32) if dtype == "bf16" else got
        want = oracle_ns(f.reshape(f.shape[0], cols), dtype, steps, QUINTIC, DEFAULT_EPS)
        err = float(np.max(np.abs(got.astype(np.float64) - want)))
        assert err <= TOL[dtype], f"tensor {i} {f.shape}: {err}"


def _compare(shapes, split_rows, S, dtype, fulls, steps=5, check=None, home=None):
    shards_host = _shards(fulls, split_rows, S, dtype)
    plan = _plan(shapes, split_rows, S, dtype, home)
    fused = _fused(plan, shards_host, dtype, steps)
    ref = _unfused(plan, shapes, shards_host, dtype, steps)
    for s in range(S):
        assert np.array_equal(fused[s].view(np.uint8), ref[s].view(np.uint8)), f"shard {s}"
    _oracle_check(fulls, split_rows, S, fused, dtype, steps, check)
    return plan, shards_host, fused


def test_square_set_uneven_shards():
    ms = routed_square_batch(True)
    fulls = [host_matrix(ms.seed, i, s) for i, s in enumerate(ms.shapes)]
    log("fused route: 16 x 1024^2 bf16, 4 uneven shards")
    _compare(ms.shapes, ms.split_rows, ms.num_shards, "bf16", fulls, check={0, 7, 15})


def _ragged_case(seed, S, dtype):
    rng = random.Random(seed)
    shapes = [(200, 333), (333, 200), (129, 257), (1, 5), (5, 1), (300, 128), (3, 40, 5), (1000, 130),
              (127, 1025), (0, 9), (6, 0), (77, 3, 7)]
    split = []
    for s in shapes:
        cuts = sorted(rng.randint(0, s[0]) for _ in range(S - 1))
        split.append([b - a for a, b in zip([0] + cuts, cuts + [s[0]])])
    std = 0.02 if dtype == "bf16" else 1.0
    fulls = [host_matrix(seed, i, s, std=std, dtype=dtype) for i, s in enumerate(shapes)]
    home = [rng.randrange(S) for _ in shapes]   # a tensor with no rows has no holder to plan from
    return shapes, split, fulls, home


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_ragged_uneven_unaligned(dtype):
    shapes, split, fulls, home = _ragged_case(31, 5, dtype)
    log(f"fused route: ragged {dtype}, 5 shards")
    _compare(shapes, split, 5, dtype, fulls, home=home)


def test_many_pieces_per_tile():
    # a tall tensor (stored rows are X columns) and a wide one, in 1-3 row
    # pieces over 64 shards: up to ~60 pieces inside one tile
    rng = random.Random(7)
    shapes = [(150, 96), (90, 300)]
    split = []
    for s in shapes:
        r = [0] * 64
        left = s[0]
        for k in range(64):
            take = min(left, rng.randint(1, 3)) if k < 63 else left
            r[k] = take
            left -= take
        split.append(r)
    fulls = [host_matrix(8, i, s) for i, s in enumerate(shapes)]
    log("fused route: many pieces per tile")
    _compare(shapes, split, 64, "bf16", fulls)


def test_staging_run_length_same_bits(monkeypatch):
    """Routed input staging in runs of several tiles (each run's band of rows
    may span many pieces) gives the bits of one tile per workgroup."""
    rng = random.Random(11)
    shapes = [(700, 300), (300, 900), (64, 2000)]
    split = []
    for s in shapes:
        r = [0] * 16
        left = s[0]
        for k in range(16):
            take = min(left, rng.randint(1, 90)) if k < 15 else left
            r[k] = take
            left -= take
        split.append(r)
    fulls = [host_matrix(12, i, s) for i, s in enumerate(shapes)]
    shards_host = _shards(fulls, split, 16, "bf16")
    plan = _plan(shapes, split, 16, "bf16")
    log("fused route: staging run lengths 1 and 5")
    monkeypatch.setenv("NS_STAGE_RUN", "1")
    one = _fused(plan, shards_host, "bf16")
    _oracle_check(fulls, split, 16, one, "bf16")
    monkeypatch.setenv("NS_STAGE_RUN", "5")
    five = _fused(plan, shards_host, "bf16")
    for s in range(16):
        assert np.array_equal(one[s].view(np.uint8), five[s].view(np.uint8)), f"shard {s}"


def test_in_place_and_zero_steps():
    shapes, split, fulls, home = _ragged_case(32, 3, "bf16")
    shards_host = _shards(fulls, split, 3, "bf16")
    plan = _plan(shapes, split, 3, "bf16", home)
    log("fused route: in place")
    ref = _fused(plan, shards_host, "bf16")
    inplace = _fused(plan, shards_host, "bf16", in_place=True)
    for a, b in zip(ref, inplace):
        assert np.array_equal(a, b)
    log("fused route: zero steps")
    zero = _fused(plan, shards_host, "bf16", steps=0)
    unf = _unfused(plan, shapes, shards_host, "bf16", steps=0)
    for a, b in zip(zero, unf):
        assert np.array_equal(a, b)
    _oracle_check(fulls, split, 3, zero, "bf16", steps=0)


def test_minimum_workspace_same_bits():
    import torch
    shapes, split, fulls, home = _ragged_case(33, 4, "bf16")
    shards_host = _shards(fulls, split, 4, "bf16")
    plan = _plan(shapes, split, 4, "bf16", home)
    need, minimum = nsq.ns_routed_workspace_bytes(plan, nsq.NS_BF16)
    assert minimum < need
    log("fused route: minimum workspace")
    full = _fused(plan, shards_host, "bf16")
    ws = torch.empty(minimum, dtype=torch.uint8, device="cuda")
    small = _fused(plan, shards_host, "bf16", workspace=ws)
    for a, b in zip(full, small):
        assert np.array_equal(a, b)
