"""GPU parity of ns_orthogonalize_batched against the fp64 oracle.

Bar: max abs error <= 2e-2 for bf16 tensors and <= 1e-4 for fp32 tensors,
element by element, on the same seeded inputs. Sizes span several 128x128
tiles with ragged tails, tall and wide orientations, 3-D tensors, and the
method's degenerate cases (zero matrix, a single row or column, zero-size
tensors, zero steps, c = 0). Also: run-to-run determinism, batch invariance
(order and company do not change a matrix's bits), and identical results with a
workspace too small for the whole batch.
"""

import numpy as np
import pytest

import newton_schulz_quintic_amd as nsq
from tests.helpers import TOL, log, oracle_ns, to_device, to_host
from workloads import CUBIC, DEFAULT_EPS, QUINTIC, host_matrix, single_fp32, square_batch

pytestmark = pytest.mark.gpu


def _run_gpu(hosts, dtype, steps=5, coeffs=QUINTIC, eps=DEFAULT_EPS, order=None, workspace=None):
    import torch
    ins = [to_device(h, dtype) for h in hosts]
    outs = [torch.empty_like(x) for x in ins]
    nsq.ns_orthogonalize_batched(ins, outs, steps=steps, coeffs=coeffs, eps=eps, order=order,
                                 workspace=workspace)
    torch.cuda.synchronize()
    return [to_host(o, dtype) for o in outs]


def _check(hosts, dtype, outs, steps=5, coeffs=QUINTIC, eps=DEFAULT_EPS, tol=None):
    tol = TOL[dtype] if tol is None else tol
    worst = 0.0
    for h, o in zip(hosts, outs):
        want = oracle_ns(h, dtype, steps, coeffs, eps)
        got = (o.astype(np.uint32) << 16).view(np.float32) if dtype == "bf16" else o
        assert got.shape == want.shape
        err = float(np.max(np.abs(got.astype(np.float64) - want))) if want.size else 0.0
        worst = max(worst, err)
        assert err <= tol, f"shape {h.shape}: max abs err {err} > {tol}"
    return worst


def test_fp32_single_matrix_quintic_and_tall():
    ms = single_fp32()
    g = host_matrix(ms.seed, 0, ms.shapes[0], std=1.0, dtype="f32")
    log("ns: fp32 64x128 quintic, and its transpose")
    hosts = [g, np.ascontiguousarray(g.T)]
    _check(hosts, "f32", _run_gpu(hosts, "f32"))


def test_fp32_cubic_thirty_steps_is_polar_factor():
    g = host_matrix(0, 0, (64, 128), std=1.0, dtype="f32")
    log("ns: fp32 64x128 cubic x30")
    out = _run_gpu([g, np.ascontiguousarray(g.T)], "f32", steps=30, coeffs=CUBIC)
    u, s, vt = np.linalg.svd(g.astype(np.float64), full_matrices=False)
    polar = u @ vt
    assert np.max(np.abs(out[0] - polar)) <= 1e-4
    assert np.max(np.abs(out[1] - polar.T)) <= 1e-4


def test_bf16_square_set_full():
    ms = square_batch()
    hosts = [host_matrix(ms.seed, i, s) for i, s in enumerate(ms.shapes)]
    log("ns: bf16 16 x 1024^2")
    worst = _check(hosts, "bf16", _run_gpu(hosts, "bf16"))
    log(f"   worst abs err {worst:.3e}")


RAGGED = [(200, 333), (333, 200), (129, 257), (1, 5), (5, 1), (64, 64), (300, 128), (3, 40, 5),
          (1000, 130), (2, 2), (127, 1025)]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_ragged_batch(dtype):
    std = 0.02 if dtype == "bf16" else 1.0
    hosts = [host_matrix(11, i, s, std=std, dtype=dtype) for i, s in enumerate(RAGGED)]
    log(f"ns: ragged batch {dtype}")
    _check(hosts, dtype, _run_gpu(hosts, dtype))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_degenerate_cases(dtype):
    import torch
    log(f"ns: degenerate cases {dtype}")
    zero = np.zeros((70, 90), dtype=np.uint16 if dtype == "bf16" else np.float32)
    small = host_matrix(12, 0, (20, 30), dtype=dtype)
    outs = _run_gpu([zero, small], dtype)
    assert not np.any(outs[0])                           # zero in, zero out (+0.0 bits)
    _check([small], dtype, outs[1:])
    # zero steps: the normalised input, transposed back
    _check([small, np.ascontiguousarray(small.T)], dtype,
           _run_gpu([small, np.ascontiguousarray(small.T)], dtype, steps=0), steps=0)
    # c = 0 (the cubic) skips the A A product
    _check([small], dtype, _run_gpu([small], dtype, steps=7, coeffs=CUBIC), steps=7, coeffs=CUBIC)
    # zero-size tensors and 1-D tensors in a batch are left alone
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    ins = [torch.empty((0, 7), dtype=tdt, device="cuda"), to_device(small, dtype),
           torch.ones((5,), dtype=tdt, device="cuda")]
    outs = [torch.empty_like(x) for x in ins]
    outs[2].fill_(3.0)
    nsq.ns_orthogonalize_batched(ins, outs)
    torch.cuda.synchronize()
    _check([small], dtype, [to_host(outs[1], dtype)])
    assert torch.all(outs[2] == 3.0)


def test_in_place_output():
    import torch
    h = host_matrix(13, 0, (256, 384))
    x = to_device(h, "bf16")
    log("ns: in place")
    nsq.ns_orthogonalize_batched([x], [x])
    torch.cuda.synchronize()
    _check([h], "bf16", [to_host(x, "bf16")])


def test_deterministic_and_batch_invariant():
    shapes = [(512, 700), (700, 512), (256, 256), (96, 1000)]
    hosts = [host_matrix(14, i, s) for i, s in enumerate(shapes)]
    log("ns: determinism / batch invariance")
    a = _run_gpu(hosts, "bf16")
    b = _run_gpu(hosts, "bf16")
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
    rev = _run_gpu(hosts[::-1], "bf16", order=[3, 1, 2, 0])[::-1]
    for x, y in zip(a, rev):
        assert np.array_equal(x, y)
    for i, h in enumerate(hosts):
        alone = _run_gpu([h], "bf16")[0]
        assert np.array_equal(alone, a[i])


def test_small_workspace_gives_same_bits():
    import torch
    shapes = [(384, 640), (256, 256), (640, 384), (128, 1024)]
    hosts = [host_matrix(15, i, s) for i, s in enumerate(shapes)]
    full = _run_gpu(hosts, "bf16")
    need, minimum = nsq.ns_workspace_bytes(shapes, nsq.NS_BF16)
    assert minimum < need
    ws = torch.empty(minimum, dtype=torch.uint8, device="cuda")
    log("ns: minimum workspace (one matrix at a time)")
    small = _run_gpu(hosts, "bf16", workspace=ws)
    for x, y in zip(full, small):
        assert np.array_equal(x, y)
    _check(hosts, "bf16", small)


def test_routed_equals_unrouted_bitwise():
    """pack -> NS on the home buffers -> unpack gives each shard exactly its rows of NS(full)."""
    import torch
    from workloads import routed_square_batch
    ms = routed_square_batch(True)
    fulls = [host_matrix(ms.seed, i, s) for i, s in enumerate(ms.shapes)]
    S = ms.num_shards
    p = nsq.ns_plan(ms.shapes, 5, S, ms.split_rows)
    plan = nsq.ns_route_plan_create(ms.shapes, S, ms.split_rows, p["home"], 2)
    q = nsq.ns_route_plan_query(plan)
    nsq.ns_route_plan_upload(plan)
    parts = [[] for _ in range(S)]
    for f, split in zip(fulls, ms.split_rows):
        for s, blk in enumerate(np.split(f, np.cumsum(split)[:-1], axis=0)):
            parts[s].append(blk.ravel())
    shards = [to_device(np.concatenate(x), "bf16") if q["shard_elems"][s] else None
              for s, x in enumerate(parts)]
    homes = [torch.empty(n, dtype=torch.bfloat16, device="cuda") if n else None for n in q["home_elems"]]
    log("ns: routed vs unrouted")
    nsq.ns_pack_shards(plan, shards, homes)
    views_in, views_out, res = [], [], []
    for i, s in enumerate(ms.shapes):
        h, off = p["home"][i], q["home_offset"][i]
        views_in.append(homes[h][off:off + s[0] * s[1]].view(s))
    res = [torch.empty_like(v) for v in views_in]
    nsq.ns_orthogonalize_batched(views_in, res, order=p["order"])
    for i, s in enumerate(ms.shapes):
        views_in[i].copy_(res[i])
    nsq.ns_unpack_shards(plan, homes, shards)
    torch.cuda.synchronize()
    direct = _run_gpu(fulls, "bf16")
    for s in range(S):
        if not q["shard_elems"][s]:
            continue
        want = []
        for i, split in enumerate(ms.split_rows):
            want.append(np.split(direct[i], np.cumsum(split)[:-1], axis=0)[s].ravel())
        assert np.array_equal(to_host(shards[s], "bf16"), np.concatenate(want))


# m > 1024: f32 B X reads the stored X^T (K-major only for K <= 1024); bf16 reads X K-major
LONG_K = [(1100, 1300), (1300, 1100), (300, 700)]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_long_k_parity(dtype):
    std = 0.02 if dtype == "bf16" else 1.0
    hosts = [host_matrix(17, i, s, std=std, dtype=dtype) for i, s in enumerate(LONG_K)]
    log(f"ns: long-K batch {dtype} {LONG_K}")
    _check(hosts, dtype, _run_gpu(hosts, dtype))


@pytest.mark.parametrize("dtype,tile", [("bf16", None), ("bf16", "256"), ("f32", None)])
def test_b_x_operand_layout_does_not_change_bits(dtype, tile, monkeypatch):
    """B X reads X either K-major (LDS transpose reads) or as the stored X^T's
    rows: the same products in the same order, so the same bits. tile "256"
    forces the 4-wave 256-tile kernel, whose calls read K-major by default."""
    std = 0.02 if dtype == "bf16" else 1.0
    shapes = [(1100, 1300), (1300, 1100), (700, 500), (64, 64)]
    hosts = [host_matrix(18, i, s, std=std, dtype=dtype) for i, s in enumerate(shapes)]
    log(f"ns: K-major vs X^T operand {dtype} tile {tile}")
    if tile:
        monkeypatch.setenv("NS_TILE", tile)
    monkeypatch.setenv("NS_KMAJOR_MAX", "0")
    stored = _run_gpu(hosts, dtype)
    monkeypatch.setenv("NS_KMAJOR_MAX", "100000")
    kmajor = _run_gpu(hosts, dtype)
    for x, y in zip(stored, kmajor):
        assert np.array_equal(x, y)


def test_tile_size_does_not_change_bits(monkeypatch):
    """The product tile (256 or 128, picked per call from the batch's size) must
    not change a matrix's bits: batch invariance across tile choices."""
    shapes = [(1024, 1024), (512, 1536), (1536, 512), (300, 700), (1100, 1300)]
    hosts = [host_matrix(16, i, s) for i, s in enumerate(shapes)]
    log("ns: 256 vs 128 product tiles")
    monkeypatch.setenv("NS_TILE", "256")
    big = _run_gpu(hosts, "bf16")
    monkeypatch.setenv("NS_TILE", "128")
    small = _run_gpu(hosts, "bf16")
    for x, y in zip(big, small):
        assert np.array_equal(x, y)


BIG_TILE_SHAPES = [(1, 300), (70, 300), (150, 400), (250, 600), (300, 700), (700, 500), (1100, 1300),
                   (1300, 1100), (512, 1536)]


@pytest.mark.parametrize("steps,coeffs", [(5, QUINTIC), (3, (2.0, -1.5, 0.0))])
def test_big_tile_kernels_give_the_same_bits(steps, coeffs, monkeypatch):
    """The bf16 256-tiles run on four waves with accumulators in fixed
    registers, or (NS_BIG_WAVES=8) on eight waves: the same MFMA over the same k
    order and the same epilogue, so the same bits, equal to the 128-tile path's
    too. Covers 1, 2, 3, 4 and 5 K stages of A A and B X (m = 1, 70, 150, 250,
    300 with the small class off), K-major and X^T operands of B X, ragged
    tails, and c = 0 (B' = a I + b A, no A A product)."""
    hosts = [host_matrix(31, i, s) for i, s in enumerate(BIG_TILE_SHAPES)]
    log(f"ns: 4-wave vs 8-wave 256 tiles, steps={steps} coeffs={coeffs}")
    monkeypatch.setenv("NS_SMALL_MAX", "0")
    monkeypatch.setenv("NS_TILE", "256")
    four = _run_gpu(hosts, "bf16", steps=steps, coeffs=coeffs)
    _check(hosts, "bf16", four, steps=steps, coeffs=coeffs)
    monkeypatch.setenv("NS_BIG_WAVES", "8")
    eight = _run_gpu(hosts, "bf16", steps=steps, coeffs=coeffs)
    monkeypatch.delenv("NS_BIG_WAVES")
    monkeypatch.setenv("NS_TILE", "128")
    small = _run_gpu(hosts, "bf16", steps=steps, coeffs=coeffs)
    for s, x, y, z in zip(BIG_TILE_SHAPES, four, eight, small):
        assert np.array_equal(x, y), s
        assert np.array_equal(x, z), s


SMALL_CLASS = [(1, 7), (7, 1), (5, 3, 4), (64, 64), (100, 1000), (1000, 100), (128, 129), (129, 128),
               (128, 128), (96, 700), (33, 4097), (2, 2), (300, 700), (127, 1025)]


@pytest.mark.parametrize("dtype,steps,coeffs", [("bf16", 5, QUINTIC), ("bf16", 1, QUINTIC), ("f32", 5, QUINTIC),
                                                ("f32", 7, CUBIC), ("bf16", 3, (2.0, -1.5, 0.0))])
def test_small_class_equals_tiled_path(dtype, steps, coeffs, monkeypatch):
    """Matrices with m <= 128 run in the small size class (one workgroup per
    matrix, every step in one kernel, padded to 128): the same 128-tile
    products in the same order as the tiled path, so the same bits, and within
    the oracle's tolerance. Mixed with tiled matrices in one call."""
    std = 0.02 if dtype == "bf16" else 1.0
    hosts = [host_matrix(23, i, s, std=std, dtype=dtype) for i, s in enumerate(SMALL_CLASS)]
    log(f"ns: small class vs tiled path {dtype} steps={steps} coeffs={coeffs}")
    monkeypatch.setenv("NS_SMALL_MAX", "0")
    tiled = _run_gpu(hosts, dtype, steps=steps, coeffs=coeffs)
    monkeypatch.delenv("NS_SMALL_MAX")
    small = _run_gpu(hosts, dtype, steps=steps, coeffs=coeffs)
    _check(hosts, dtype, small, steps=steps, coeffs=coeffs)
    for s, x, y in zip(SMALL_CLASS, tiled, small):
        assert np.array_equal(x, y), s


def test_small_class_many_random_shapes():
    """A many-small-style batch (rows and cols log-uniform in [8, 600], most with
    m <= 128) against the oracle, and bit-identical to the tiled path."""
    import os
    rng = np.random.default_rng(29)
    shapes = [tuple(int(round(np.exp(rng.uniform(np.log(8), np.log(600))))) for _ in range(2)) for _ in range(40)]
    hosts = [host_matrix(29, i, s) for i, s in enumerate(shapes)]
    log(f"ns: 40 random small shapes, {sum(min(s) <= 128 for s in shapes)} in the small class")
    small = _run_gpu(hosts, "bf16")
    _check(hosts, "bf16", small)
    os.environ["NS_SMALL_MAX"] = "0"
    try:
        tiled = _run_gpu(hosts, "bf16")
    finally:
        del os.environ["NS_SMALL_MAX"]
    for s, x, y in zip(shapes, tiled, small):
        assert np.array_equal(x, y), s


def test_input_range_large_and_tiny_magnitudes():
    """Inputs of large magnitude within the documented range (||G||_F^2 and
    G G^T within fp32) match the oracle; past it, every output is NaN rather
    than zeros. Scale matters only through eps, so a scaled input gives the
    scaled-input oracle's result."""
    import torch
    base = host_matrix(61, 0, (300, 1024), std=1.0, dtype="f32")
    ok = [base * np.float32(1e15), base * np.float32(1e-15)]   # ||G|| ~ 5.5e17 and 5.5e-13
    for h in ok:
        log(f"ns: f32 300x1024 at scale {float(np.abs(h).max()):.1e}")
        _check([h], "f32", _run_gpu([h], "f32"))
    big = [base * np.float32(1e18)]                             # ||G||^2 ~ 3e41: past fp32
    log("ns: f32 300x1024 past the fp32 range of ||G||^2")
    out = _run_gpu(big, "f32")[0]
    assert np.all(np.isnan(out))
    bf = host_matrix(62, 0, (64, 2048), std=1.0)                # bf16 bits of N(0, 1)
    big_bf = (bf.astype(np.uint32) + (60 << 7)).astype(np.uint16)   # x 2^60 (exponent + 60): ||G||^2 ~ 1.7e41
    log("ns: bf16 64x2048 past the fp32 range of ||G||^2")
    got = _run_gpu([big_bf], "bf16")[0]
    vals = (got.astype(np.uint32) << 16).view(np.float32)
    assert np.all(np.isnan(vals))
    del torch


def test_side_stream_without_workspace_keeps_its_memory():
    """A call on a side stream with no workspace given: the library's
    workspace, dropped by the caller at once, is not handed to new work on
    the current stream while the call may still run there, and the outputs
    match the oracle. A spin kernel queued ahead on the side stream keeps the
    call pending while the same-size allocation is made."""
    import torch
    hosts = [host_matrix(71, i, (1024, 1536)) for i in range(3)]
    ins = [to_device(h, "bf16") for h in hosts]
    outs = [torch.empty_like(x) for x in ins]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    log("ns: bf16 3 x 1024x1536 on a side stream, workspace dropped")
    with torch.cuda.stream(side):
        torch.cuda._sleep(50_000_000)   # spin (25 ms to 0.5 s, by the counter's clock) ahead of the call
    ws = nsq.ns_orthogonalize_batched(ins, outs, stream=side)
    held, nbytes = ws.data_ptr(), ws.numel()
    del ws
    other = torch.empty(nbytes, dtype=torch.uint8, device=ins[0].device)
    assert other.data_ptr() != held, "a block still in use on the side stream was handed out"
    other.fill_(0xFF)
    side.synchronize()
    torch.cuda.synchronize()
    _check(hosts, "bf16", [to_host(o, "bf16") for o in outs])


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_staging_run_length_does_not_change_bits(dtype, monkeypatch):
    """Input staging walks runs of tiles per workgroup (one tile for small calls,
    several for large ones). Each tile's copy and sum of squares is the same
    work either way, so the run length must not change a bit: wide, tall, 3-D,
    ragged edges and a single row, with runs of 1, 3 (ragged run tails) and 16
    tiles, for 5 steps and for 0 (the scale-out path walks the same runs)."""
    shapes = [(300, 700), (700, 300), (5, 60, 40), (1, 900), (1024, 1024), (129, 1100)]
    hosts = [host_matrix(41, i, s, dtype=dtype) for i, s in enumerate(shapes)]
    log(f"ns: staging run lengths, {dtype}")
    for steps in (5, 0):
        monkeypatch.setenv("NS_STAGE_RUN", "1")
        ref = _run_gpu(hosts, dtype, steps=steps)
        _check(hosts, dtype, ref, steps=steps)
        for run in ("3", "16"):
            monkeypatch.setenv("NS_STAGE_RUN", run)
            got = _run_gpu(hosts, dtype, steps=steps)
            for h, x, y in zip(hosts, ref, got):
                assert np.array_equal(x.view(np.uint8), y.view(np.uint8)), f"{h.shape} run {run} steps {steps}"
