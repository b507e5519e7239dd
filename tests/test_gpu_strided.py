"""GPU parity of ns_orthogonalize_strided: NS on sub-blocks of fused weights.

Bar: bit-identical to ns_orthogonalize_batched on contiguous copies of the
blocks, within the oracle tolerance, and nothing outside the output views is
written. Cases: Q/K/V row blocks of a (3h, h) weight, column blocks of an
(h, 3h) weight (row stride 3h), odd widths (no 16-byte accesses), tall blocks,
in place, fp32.
"""

import numpy as np
import pytest

import newton_schulz_quintic_amd as nsq
from tests.helpers import TOL, log, oracle_ns, to_device, to_host
from workloads import host_matrix

pytestmark = pytest.mark.gpu


def _contiguous_ns(blocks_host, dtype):
    import torch
    ins = [to_device(np.ascontiguousarray(b), dtype) for b in blocks_host]
    outs = [torch.empty_like(x) for x in ins]
    nsq.ns_orthogonalize_batched(ins, outs)
    torch.cuda.synchronize()
    return [to_host(o, dtype) for o in outs]


def _run(fused_host, cuts, axis, dtype, in_place=False):
    import torch
    w = to_device(fused_host, dtype)
    sentinel = float("nan")
    o = w if in_place else torch.full_like(w, sentinel)
    views_in, views_out, blocks = [], [], []
    for lo, hi in cuts:
        sl = (slice(lo, hi), slice(None)) if axis == 0 else (slice(None), slice(lo, hi))
        views_in.append(w[sl])
        views_out.append(o[sl])
        blocks.append(fused_host[sl])
    want = _contiguous_ns(blocks, dtype)
    nsq.ns_orthogonalize_strided(views_in, views_out)
    torch.cuda.synchronize()
    got_all = to_host(o, dtype)
    for (lo, hi), wnt, blk in zip(cuts, want, blocks):
        sl = (slice(lo, hi), slice(None)) if axis == 0 else (slice(None), slice(lo, hi))
        got = got_all[sl]
        assert np.array_equal(np.ascontiguousarray(got), wnt)
        ref = oracle_ns(np.ascontiguousarray(blk), dtype, 5, (3.4445, -4.7750, 2.0315), 1e-7)
        g = (got.astype(np.uint32) << 16).view(np.float32) if dtype == "bf16" else got
        assert float(np.max(np.abs(g.astype(np.float64) - ref))) <= TOL[dtype]
    if not in_place:
        covered = np.zeros(got_all.shape, bool)
        for lo, hi in cuts:
            if axis == 0:
                covered[lo:hi, :] = True
            else:
                covered[:, lo:hi] = True
        rest = got_all[~covered]
        if dtype == "bf16":
            rest = (rest.astype(np.uint32) << 16).view(np.float32)
        assert np.all(np.isnan(rest))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_qkv_row_blocks(dtype):
    h = 384
    std = 0.02 if dtype == "bf16" else 1.0
    fused = host_matrix(51, 0, (3 * h, h), std=std, dtype=dtype)
    log(f"strided: QKV row blocks {dtype}")
    _run(fused, [(0, h), (h, 2 * h), (2 * h, 3 * h)], 0, dtype)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_qkv_column_blocks(dtype):
    h = 320
    std = 0.02 if dtype == "bf16" else 1.0
    fused = host_matrix(52, 0, (h, 3 * h), std=std, dtype=dtype)
    log(f"strided: QKV column blocks {dtype}")
    _run(fused, [(0, h), (h, 2 * h), (2 * h, 3 * h)], 1, dtype)


def test_odd_widths_tall_blocks_and_gaps():
    # column blocks of odd widths with unused columns between them; the
    # 300-row, 77-column block is tall (stored rows are X columns)
    fused = host_matrix(53, 0, (300, 420), std=0.02)
    log("strided: odd widths, tall blocks, gaps")
    _run(fused, [(0, 77), (80, 157), (161, 420)], 1, "bf16")


def test_in_place_blocks():
    fused = host_matrix(54, 0, (256, 3 * 200), std=0.02)
    log("strided: in place")
    _run(fused, [(0, 200), (200, 400), (400, 600)], 1, "bf16", in_place=True)
