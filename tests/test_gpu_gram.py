"""GPU parity of ns_orthogonalize_gram (Gram-space NS, fp32) against the oracle.

Bar: max abs error <= 1e-4 against the fp64 Gram-space oracle for fp32
tensors and <= 2e-2 for bf16 tensors (their output is rounded to bf16 once),
on ragged wide / tall / 3-D sets, a short-and-wide case (m << n, where the
Gram space pays), the trace ridge, steps 0 and 1, and c = 0. With ridge 0 the
oracle is the standard iteration too (the reformulation is exact).
"""

import numpy as np
import pytest

import newton_schulz_quintic_amd as nsq
from oracle import ns as ons
from tests.helpers import TOL, host_to_f64, log, oracle_ns, to_device, to_host
from workloads import CUBIC, DEFAULT_EPS, QUINTIC, host_matrix

pytestmark = pytest.mark.gpu

SHAPES = [(200, 333), (333, 200), (129, 257), (64, 64), (3, 40, 5), (1, 9), (9, 1), (256, 256), (96, 700)]


def _gram_gpu(hosts, dtype, steps=5, coeffs=QUINTIC, ridge=0.0):
    import torch
    ins = [to_device(h, dtype) for h in hosts]
    outs = [torch.empty_like(x) for x in ins]
    nsq.ns_orthogonalize_gram(ins, outs, steps=steps, coeffs=coeffs, eps=DEFAULT_EPS, ridge=ridge)
    torch.cuda.synchronize()
    return [to_host(o, dtype) for o in outs]


def _check(hosts, outs, dtype, steps=5, coeffs=QUINTIC, ridge=0.0):
    a, b, c = (float(np.float32(x)) for x in coeffs)
    worst = 0.0
    for h, o in zip(hosts, outs):
        want = ons.newton_schulz_gram(host_to_f64(h, dtype), steps, a, b, c, float(np.float32(DEFAULT_EPS)),
                                      ridge=float(np.float32(ridge)))
        got = (o.astype(np.uint32) << 16).view(np.float32) if dtype == "bf16" else o
        err = float(np.max(np.abs(got.astype(np.float64) - want)))
        worst = max(worst, err)
        assert err <= TOL[dtype], f"{h.shape}: {err}"
    return worst


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_ragged_set(dtype):
    std = 0.02 if dtype == "bf16" else 1.0
    hosts = [host_matrix(61, i, s, std=std, dtype=dtype) for i, s in enumerate(SHAPES)]
    log(f"gram: ragged set {dtype}")
    outs = _gram_gpu(hosts, dtype)
    log(f"   worst {_check(hosts, outs, dtype):.3e}")
    if dtype == "f32":
        # ridge 0: the standard iteration's oracle agrees as well
        for h, o in zip(hosts, outs):
            assert np.max(np.abs(o - oracle_ns(h, dtype, 5, QUINTIC, DEFAULT_EPS))) <= TOL[dtype]


def test_short_and_wide_and_ridge():
    hosts = [host_matrix(62, 0, (128, 4096), std=1.0, dtype="f32"),
             host_matrix(62, 1, (2048, 256), std=1.0, dtype="f32")]
    log("gram: m << n, ridge 0 and 1e-3")
    _check(hosts, _gram_gpu(hosts, "f32"), "f32")
    _check(hosts, _gram_gpu(hosts, "f32", ridge=1e-3), "f32", ridge=1e-3)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_steps_and_cubic(dtype):
    std = 0.02 if dtype == "bf16" else 1.0
    hosts = [host_matrix(63, i, s, std=std, dtype=dtype) for i, s in enumerate([(70, 90), (150, 40)])]
    log(f"gram: steps 0, 1 and the cubic {dtype}")
    _check(hosts, _gram_gpu(hosts, dtype, steps=0), dtype, steps=0)
    _check(hosts, _gram_gpu(hosts, dtype, steps=1), dtype, steps=1)
    _check(hosts, _gram_gpu(hosts, dtype, steps=7, coeffs=CUBIC), dtype, steps=7, coeffs=CUBIC)
    zero = np.zeros((40, 60), dtype=np.uint16 if dtype == "bf16" else np.float32)
    assert not np.any(_gram_gpu([zero], dtype)[0])


def test_staging_run_length_same_bits(monkeypatch):
    """Gram-space staging widens bf16 inputs to fp32 tile by tile; runs of
    several tiles per workgroup must give the bits of one tile each."""
    hosts = [host_matrix(52, i, s) for i, s in enumerate(SHAPES)]
    log("gram: staging run lengths 1 and 3")
    monkeypatch.setenv("NS_STAGE_RUN", "1")
    one = _gram_gpu(hosts, "bf16")
    _check(hosts, one, "bf16")
    monkeypatch.setenv("NS_STAGE_RUN", "3")
    three = _gram_gpu(hosts, "bf16")
    for h, x, y in zip(hosts, one, three):
        assert np.array_equal(x.view(np.uint8), y.view(np.uint8)), f"{h.shape}"
