"""GPU parity at the full sizes of the measured matrix sets.

Every matrix of the set runs through one ns_orthogonalize_batched call, in the
launch configuration bench.py times. Then:

* every output is checked for properties that hold at any size: all finite,
  and largest singular value (power iteration, fp32) <= max of p on [0, 1]
  (about 1.2024) plus a bf16 margin;
* a sample (one matrix per distinct shape for the dense-transformer set; the
  MoE shapes plus a seeded sample of the random shapes for the many-small set)
  is compared element by element with the fp64 oracle (max abs <= 2e-2). The
  oracle gets the exact bf16 inputs, copied back from the device.
"""

import numpy as np
import pytest

import newton_schulz_quintic_amd as nsq
from tests.helpers import TOL, log, oracle_ns
from workloads import DEFAULT_EPS, QUINTIC, dense_transformer, device_matrix, many_small

pytestmark = pytest.mark.gpu

SIGMA_BOUND = 1.2024 * 1.03   # max of the quintic on [0, 1], plus a bf16 margin


def _to_host_bits(t):
    import torch
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def _sigma_max(t, iters=30):
    import torch
    x = t.float()
    if x.shape[0] > x.shape[1]:
        x = x.t()
    v = torch.randn(x.shape[1], device=x.device, generator=torch.Generator(device=x.device).manual_seed(0))
    for _ in range(iters):
        v = x.t().mv(x.mv(v))
        v = v / v.norm()
    return float(x.mv(v).norm())


def _run_set(ms, sample_idx):
    import torch
    log(f"large: generating {ms.name} ({ms.n} matrices) on the device")
    ins = [device_matrix(ms.seed, i, s, std=ms.std) for i, s in enumerate(ms.shapes)]
    sample_in = {i: _to_host_bits(ins[i]) for i in sample_idx}
    order = nsq.ns_plan(ms.shapes, 5, 1)["order"]
    log(f"large: NS over {ms.n} matrices (in place)")
    nsq.ns_orthogonalize_batched(ins, ins, steps=5, coeffs=QUINTIC, eps=DEFAULT_EPS, order=order)
    torch.cuda.synchronize()
    log("large: properties of every output")
    worst_sigma = 0.0
    for i, y in enumerate(ins):
        assert bool(torch.isfinite(y).all()), f"matrix {i} {ms.shapes[i]}: non-finite output"
        sig = _sigma_max(y)
        worst_sigma = max(worst_sigma, sig)
        assert sig <= SIGMA_BOUND, f"matrix {i} {ms.shapes[i]}: sigma_max {sig}"
    log(f"large: worst sigma_max {worst_sigma:.4f}")
    sample_out = {i: _to_host_bits(ins[i]) for i in sample_idx}
    del ins
    torch.cuda.empty_cache()
    worst = 0.0
    for i in sample_idx:
        log(f"large: oracle for matrix {i} {ms.shapes[i]}")
        want = oracle_ns(sample_in[i], "bf16", 5, QUINTIC, DEFAULT_EPS)
        got = (sample_out[i].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        err = float(np.max(np.abs(got - want)))
        worst = max(worst, err)
        assert err <= TOL["bf16"], f"matrix {i} {ms.shapes[i]}: max abs err {err}"
    log(f"large: worst sampled max abs err {worst:.3e}")


def test_dense_transformer_full_set():
    ms = dense_transformer()
    first = {}
    for i, s in enumerate(ms.shapes):
        first.setdefault(s, i)
    _run_set(ms, sorted(first.values()))          # q, k, gate, down of layer 0


def test_many_small_full_set():
    ms = many_small()
    rng = np.random.default_rng(77)
    sample = sorted(set(rng.choice(3000, size=16, replace=False).tolist()) | {3000, 3001, 3002})
    _run_set(ms, sample)


def test_long_thin_matrix():
    import torch
    from workloads import host_matrix
    from tests.helpers import to_device, to_host
    h = host_matrix(31, 0, (128, 131072))
    x = to_device(h, "bf16")
    y = torch.empty_like(x)
    log("large: 128 x 131072")
    nsq.ns_orthogonalize_batched([x], [y])
    torch.cuda.synchronize()
    want = oracle_ns(h, "bf16", 5, QUINTIC, DEFAULT_EPS)
    got = (to_host(y, "bf16").astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    assert float(np.max(np.abs(got - want))) <= TOL["bf16"]


def test_largest_accepted_matrix_structured():
    """The largest bf16 matrix with m = 256 the size limits accept (n =
    2,796,032; one more padded tile and the kept X^T would reach 2^31 bytes),
    wide and tall. Its rows are orthogonal with equal norms (a Sylvester-
    Hadamard block tiled along n, times seeded column signs), so every singular
    value of X0 is 1/sqrt(m) and the iteration returns kappa * G with
    kappa = p^5(1/sqrt(m)) / sqrt(n), p the step polynomial on singular values.
    kappa * sqrt(n) does not depend on n: it is read off the oracle's output for
    the same structure at n = 2048. Every output element, times sqrt(n) (the
    unit scale of the other bf16 parity tests), must be within 2e-2 of it."""
    import torch
    from workloads import bf16_bits_to_f32, orthogonal_rows_bits
    m, n, n_small, seed = 256, 2796032, 2048, 91
    g_small = orthogonal_rows_bits(m, n_small, seed)
    want = oracle_ns(g_small, "bf16", 5, QUINTIC, DEFAULT_EPS)
    ratio = want / bf16_bits_to_f32(g_small).astype(np.float64)
    assert float(ratio.max() - ratio.min()) <= 1e-12 * float(np.abs(ratio).max())   # kappa * G exactly
    unit = float(ratio.mean()) * np.sqrt(n_small)
    big = orthogonal_rows_bits(m, n, seed)
    x = torch.from_numpy(big.view(np.int16)).view(torch.bfloat16).cuda()
    del big
    for tall in (False, True):
        if tall:
            x = x.t().contiguous()
        log(f"large: structured {tuple(x.shape)} bf16, the largest accepted size")
        y = torch.empty_like(x)
        nsq.ns_orthogonalize_batched([x], [y], steps=5, coeffs=QUINTIC, eps=DEFAULT_EPS)
        torch.cuda.synchronize()
        err = float((y.float() * np.sqrt(n) - unit * x.float()).abs().max())
        log(f"large: max abs err (sqrt(n) scale) {err:.3e}")
        assert err <= TOL["bf16"], f"{tuple(x.shape)}: {err}"
        del y
    del x
    torch.cuda.empty_cache()
