"""GPU checks of wave dispatch (ns_orthogonalize_waves).

Bar: every wave output within the bf16 tolerance of the fp64 oracle,
element by element, and bit-identical to ns_orthogonalize_batched on the same
tensors; each wave waits for its ready event: inputs written on another
stream after a long run of unrelated work, with an event per wave, come out
exactly as when they were ready from the start (and within the oracle's
tolerance).
"""

import numpy as np
import pytest

import newton_schulz_quintic_amd as nsq
from tests.helpers import TOL, host_to_f64, log, oracle_ns, to_device, to_host
from workloads import host_matrix

COEFFS = (3.4445, -4.7750, 2.0315)


def _check_oracle(hosts, outs):
    for i, (h, o) in enumerate(zip(hosts, outs)):
        want = oracle_ns(h, "bf16", 5, COEFFS, 1e-7)
        got = host_to_f64(to_host(o, "bf16"), "bf16").reshape(want.shape)
        err = float(np.max(np.abs(got - want))) if want.size else 0.0
        assert err <= TOL["bf16"], (i, SHAPES[i], err)

pytestmark = pytest.mark.gpu

SHAPES = [(200, 333), (333, 200), (129, 257), (64, 64), (300, 128), (3, 40, 5), (1000, 130), (127, 1025),
          (256, 256), (96, 700)]


def _batched(hosts):
    import torch
    ins = [to_device(h, "bf16") for h in hosts]
    outs = [torch.empty_like(x) for x in ins]
    nsq.ns_orthogonalize_batched(ins, outs)
    torch.cuda.synchronize()
    return [to_host(o, "bf16") for o in outs]


def test_waves_bit_identical_to_batched():
    import torch
    hosts = [host_matrix(41, i, s) for i, s in enumerate(SHAPES)]
    want = _batched(hosts)
    wave_of, num = nsq.ns_wave_plan(SHAPES, 4)
    assert num == 3
    ins = [to_device(h, "bf16") for h in hosts]
    outs = [torch.empty_like(x) for x in ins]
    log("waves: 3 waves, no events")
    nsq.ns_orthogonalize_waves(ins, outs, wave_of, num)
    torch.cuda.synchronize()
    _check_oracle(hosts, outs)
    for w, o in zip(want, outs):
        assert np.array_equal(w, to_host(o, "bf16"))
    # a tensor left out of every wave is untouched
    outs2 = [torch.zeros_like(x) for x in ins]
    skip = list(wave_of)
    skip[0] = -1
    nsq.ns_orthogonalize_waves(ins, outs2, skip, num)
    torch.cuda.synchronize()
    assert not torch.any(outs2[0])
    assert np.array_equal(want[1], to_host(outs2[1], "bf16"))


def test_waves_wait_for_their_events():
    import torch
    hosts = [host_matrix(42, i, s) for i, s in enumerate(SHAPES)]
    want = _batched(hosts)
    wave_of, num = nsq.ns_wave_plan(SHAPES, 3)
    src = [to_device(h, "bf16") for h in hosts]
    ins = [torch.zeros_like(x) for x in src]       # filled later, on the producer stream
    outs = [torch.empty_like(x) for x in ins]
    ws_need, _ = nsq.ns_workspace_bytes(SHAPES, nsq.NS_BF16)
    ws = torch.empty(ws_need, dtype=torch.uint8, device="cuda")
    a = torch.randn(2048, 2048, device="cuda")
    torch.cuda.synchronize()
    producer, consumer = torch.cuda.Stream(), torch.cuda.Stream()
    events = [torch.cuda.Event() for _ in range(num)]
    log("waves: inputs produced late on another stream, one event per wave")
    with torch.cuda.stream(producer):
        for w in range(num):
            for _ in range(10):                    # unrelated work before this wave's inputs exist
                a = torch.tanh(a @ a * 1e-3)
            for i in range(len(SHAPES)):
                if wave_of[i] == w:
                    ins[i].copy_(src[i])
            events[w].record(producer)
    nsq.ns_orthogonalize_waves(ins, outs, wave_of, num, ready_events=events, workspace=ws,
                               stream=consumer)
    torch.cuda.synchronize()
    _check_oracle(hosts, outs)
    for w, o in zip(want, outs):
        assert np.array_equal(w, to_host(o, "bf16"))
