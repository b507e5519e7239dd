"""GPU check of the no-allocation entry point (ns_orthogonalize_batched_noalloc).

Bar: on two calls in a row through the C ABI, the second with a smaller
input, every output is bit-identical to ns_orthogonalize_batched's on the
same tensors and within the fp64 oracle's tolerance (2e-2 bf16, 1e-4 f32).
A set whose largest tensor needs more than the library's 64 MiB scratch is
refused with NS_ERR_WORKSPACE before anything runs, leaving the output as it
was. Also run after the other GPU tests: the array keeps earlier calls'
contents, which must not leak into a result.
"""

import numpy as np
import pytest

import newton_schulz_quintic_amd as nsq
from tests.helpers import TOL, log, oracle_ns, to_device, to_host
from workloads import QUINTIC, host_matrix

pytestmark = pytest.mark.gpu


def _pair(shapes, dtype, seed):
    import torch
    std = 0.02 if dtype == "bf16" else 1.0
    hosts = [host_matrix(seed, i, s, std=std, dtype=dtype) for i, s in enumerate(shapes)]
    ins = [to_device(h, dtype) for h in hosts]
    want = [torch.empty_like(x) for x in ins]
    nsq.ns_orthogonalize_batched(ins, want)
    got = [torch.full_like(x, 7.0) for x in ins]     # stale values the call must overwrite
    nsq.ns_orthogonalize_batched_noalloc(ins, got)
    torch.cuda.synchronize()
    for s, h, w, g in zip(shapes, hosts, want, got):
        gh, wh = to_host(g, dtype), to_host(w, dtype)
        assert np.array_equal(gh, wh), s
        ref = oracle_ns(h, dtype, 5, QUINTIC, 1e-7)
        val = (gh.astype(np.uint32) << 16).view(np.float32) if dtype == "bf16" else gh
        err = float(np.max(np.abs(val.astype(np.float64) - ref))) if ref.size else 0.0
        assert err <= TOL[dtype], (s, err)


def test_noalloc_matches_batched_two_calls():
    nsq.ns_noalloc_init()
    nsq.ns_noalloc_init()           # idempotent
    first = [(1024, 1024), (1024, 1024), (1024, 1024), (1000, 130), (129, 257), (64, 700), (3, 40, 5),
             (2048, 1024)]
    log(f"noalloc: call 1, bf16 {first}")
    _pair(first, "bf16", 51)
    second = [(200, 333), (96, 64), (5, 1)]
    log(f"noalloc: call 2 (smaller), bf16 {second}")
    _pair(second, "bf16", 52)
    log("noalloc: call 3, f32")
    _pair([(300, 200), (64, 128)], "f32", 53)


def test_noalloc_more_than_scratch_in_groups():
    # 8 x 1024^2 needs about 71 MiB at once: the call runs in groups that fit
    nsq.ns_noalloc_init()
    shapes = [(1024, 1024)] * 8
    log("noalloc: 8 x 1024^2 in groups")
    _pair(shapes, "bf16", 54)


def test_noalloc_rejects_a_tensor_larger_than_scratch():
    import torch
    nsq.ns_noalloc_init()
    x = torch.zeros(4096, 4096, dtype=torch.bfloat16, device="cuda")
    y = torch.full_like(x, 3.0)
    log("noalloc: 4096^2 needs more than 64 MiB: refused")
    with pytest.raises(nsq.NSError) as e:
        nsq.ns_orthogonalize_batched_noalloc([x], [y])
    assert e.value.name == "NS_ERR_WORKSPACE"
    torch.cuda.synchronize()
    assert bool(torch.all(y == 3.0))
