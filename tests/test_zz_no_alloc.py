"""GPU check of the no-allocation entry point (ns_orthogonalize_batched_noalloc).

Bar: on two calls in a row through the C ABI, the second with a smaller
input, every output is bit-identical to ns_orthogonalize_batched's on the
same tensors and within the fp64 oracle's tolerance (2e-2 bf16, 1e-4 f32).
A set whose largest tensor needs more than the library's 64 MiB scratch is
refused with NS_ERR_WORKSPACE before anything runs, leaving the output as it
was. Also run after the other GPU tests: the array keeps earlier calls'
contents, which must not leak into a result. A call captured into a graph
replays right after other calls have reused the staging and the array.
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


def test_noalloc_call_captured_in_a_graph_replays_right():
    """A no-allocation call captured into a HIP graph (torch.cuda.CUDAGraph)
    and replayed three times, with eager calls of the library on other
    tensors and synchronisations between the replays (they reuse the
    ordinary table staging and the scratch array the graph also uses): every
    replay overwrites stale outputs with the eager batched call's bits, which
    are within the oracle's tolerance."""
    import torch
    nsq.ns_noalloc_init()
    shapes = [(512, 768), (300, 200), (96, 1000)]
    hosts = [host_matrix(55, i, s) for i, s in enumerate(shapes)]
    ins = [to_device(h, "bf16") for h in hosts]
    want = [torch.empty_like(x) for x in ins]
    nsq.ns_orthogonalize_batched(ins, want)
    outs = [torch.empty_like(x) for x in ins]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):                    # one eager run on a side stream before capture
        nsq.ns_orthogonalize_batched_noalloc(ins, outs)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    log(f"noalloc: capture bf16 {shapes} into a graph")
    with torch.cuda.graph(graph):
        nsq.ns_orthogonalize_batched_noalloc(ins, outs)
    other_shapes = [(700, 500), (64, 64), (1024, 1024)]
    other = [to_device(host_matrix(56, i, s), "bf16") for i, s in enumerate(other_shapes)]
    other_out = [torch.empty_like(x) for x in other]
    wanted = [to_host(w, "bf16") for w in want]
    for rep in range(3):
        for o in outs:
            o.fill_(7.0)                             # stale values the replay must overwrite
        torch.cuda.synchronize()
        log(f"noalloc: replay {rep}")
        graph.replay()
        torch.cuda.synchronize()
        for s, o, w in zip(shapes, outs, wanted):
            assert np.array_equal(to_host(o, "bf16"), w), (rep, s)
        nsq.ns_orthogonalize_batched_noalloc(other, other_out)   # eager work between the replays
        nsq.ns_orthogonalize_batched(other, other_out)
        torch.cuda.synchronize()
    for s, h, w in zip(shapes, hosts, wanted):
        ref = oracle_ns(h, "bf16", 5, QUINTIC, 1e-7)
        val = (w.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        assert float(np.max(np.abs(val - ref))) <= TOL["bf16"], s
