"""Pins for the oracle Newton-Schulz (float64).

The closed form: if X0 = U S V^T then each step maps every singular value s to
p(s) = a s + b s^3 + c s^5 and keeps U and V, so after k steps
X_k = U p^k(S) V^T. This is computed here by an independent route (an SVD and
a scalar iteration), and the special cases below reduce to it.
"""

import numpy as np
import pytest

from oracle import ns
from workloads import CUBIC, QUINTIC, host_matrix

A, B, C = QUINTIC
EPS = 1e-7


def _p(s, a, b, c):
    return a * s + b * s ** 3 + c * s ** 5


def _closed_form(g, steps, a, b, c, eps):
    x = g.reshape(g.shape[0], -1)
    u, s, vt = np.linalg.svd(x, full_matrices=False)
    s = s / (np.sqrt(np.sum(s * s)) + eps)        # ||X||_F = sqrt(sum s^2)
    for _ in range(steps):
        s = _p(s, a, b, c)
    return ((u * s) @ vt).reshape(g.shape)


def test_bf16_bits_hand_values():
    bits = np.array([0x3F80, 0xC000, 0x3F81, 0x3E80, 0x0000, 0x8000, 0x7F80, 0xFF80, 0x0001],
                    dtype=np.uint16)
    v = ns.bf16_bits_to_f64(bits)
    assert v[0] == 1.0 and v[1] == -2.0 and v[2] == 1.0078125 and v[3] == 0.25
    assert v[4] == 0.0 and v[5] == 0.0 and np.signbit(v[5])
    assert np.isposinf(v[6]) and np.isneginf(v[7])
    assert v[8] == 2.0 ** -133


@pytest.mark.parametrize("shape", [(8, 13), (13, 8), (16, 16), (5, 3, 4), (1, 7), (7, 1)])
@pytest.mark.parametrize("coeffs,steps", [(QUINTIC, 5), (QUINTIC, 1), (CUBIC, 7), ((2.0, -1.5, 0.5), 3)])
def test_matches_svd_closed_form(shape, coeffs, steps):
    # fixed integer seed per case (no hash(): str hashing changes per process)
    rng = np.random.default_rng([int(np.prod(shape)), len(shape), shape[0], steps])
    g = rng.standard_normal(shape)
    got = ns.newton_schulz(g, steps, *coeffs, EPS)
    want = _closed_form(g, steps, *coeffs, EPS)
    assert got.shape == g.shape
    assert np.max(np.abs(got - want)) < 1e-12


def test_tall_is_transpose_of_wide():
    g = np.random.default_rng(3).standard_normal((40, 17))
    tall = ns.newton_schulz(g, 5, A, B, C, EPS)
    wide = ns.newton_schulz(g.T.copy(), 5, A, B, C, EPS)
    assert np.max(np.abs(tall - wide.T)) < 1e-14


def test_rank_one():
    rng = np.random.default_rng(4)
    u, v = rng.standard_normal(9), rng.standard_normal(21)
    g = np.outer(u, v)
    nrm = np.linalg.norm(u) * np.linalg.norm(v)
    s = nrm / (nrm + EPS)
    for _ in range(5):
        s = _p(s, A, B, C)
    want = s * np.outer(u / np.linalg.norm(u), v / np.linalg.norm(v))
    assert np.max(np.abs(ns.newton_schulz(g, 5, A, B, C, EPS) - want)) < 1e-13


def test_orthonormal_rows():
    # Q with orthonormal rows: ||Q||_F = sqrt(m), so X0 = Q / sqrt(m) and X_k = p^k(1/sqrt(m)) Q.
    m, n = 64, 128
    q, _ = np.linalg.qr(np.random.default_rng(5).standard_normal((n, m)))
    Q = q.T
    s = 1.0 / (np.sqrt(m) + EPS)
    for _ in range(5):
        s = _p(s, A, B, C)
    assert np.max(np.abs(ns.newton_schulz(Q, 5, A, B, C, EPS) - s * Q)) < 1e-14


def test_zero_stays_zero():
    z = np.zeros((6, 10))
    assert np.all(ns.newton_schulz(z, 5, A, B, C, EPS) == 0.0)


def test_cubic_converges_to_polar_factor():
    g = host_matrix(0, 0, (64, 128), std=1.0, dtype="f32").astype(np.float64)
    u, s, vt = np.linalg.svd(g, full_matrices=False)
    assert s[-1] / np.sqrt(np.sum(s * s)) > 0.03          # smallest singular value of X0
    got = ns.newton_schulz(g, 30, *CUBIC, EPS)
    assert np.max(np.abs(got - u @ vt)) < 1e-12
    # and its transpose (tall path)
    got_t = ns.newton_schulz(g.T.copy(), 30, *CUBIC, EPS)
    assert np.max(np.abs(got_t - (u @ vt).T)) < 1e-12


def test_quintic_singular_values_bounded():
    # p maps [0, 1] into [0, pmax] and [0, pmax] into itself, with pmax = max of p on [0, 1].
    grid = np.linspace(0.0, 1.0, 200001)
    pmax = np.max(_p(grid, A, B, C))
    assert 1.2023 < pmax < 1.2025
    wide = np.linspace(0.0, pmax, 200001)
    assert np.max(_p(wide, A, B, C)) <= pmax + 1e-9 and np.min(_p(wide, A, B, C)) >= 0.0
    for seed, shape in [(0, (64, 128)), (1, (50, 50)), (2, (200, 30))]:
        g = np.random.default_rng(seed).standard_normal(shape)
        s = np.linalg.svd(ns.newton_schulz(g, 5, A, B, C, EPS), compute_uv=False)
        assert s.max() <= pmax + 1e-12


def test_ndim_view_and_errors():
    g = np.random.default_rng(6).standard_normal((4, 3, 5))
    got = ns.newton_schulz(g, 5, A, B, C, EPS)
    assert got.shape == (4, 3, 5)
    assert np.max(np.abs(got - _closed_form(g, 5, A, B, C, EPS))) < 1e-12
    with pytest.raises(ValueError):
        ns.newton_schulz(np.ones(5), 5, A, B, C, EPS)


def test_zero_steps_is_normalised_input():
    g = np.random.default_rng(8).standard_normal((5, 9))
    got = ns.newton_schulz(g, 0, A, B, C, EPS)
    assert np.max(np.abs(got - g / (np.linalg.norm(g) + EPS))) < 1e-15


@pytest.mark.parametrize("shape", [(8, 13), (13, 8), (16, 16), (5, 3, 4), (1, 7), (24, 64)])
@pytest.mark.parametrize("coeffs,steps", [(QUINTIC, 5), (CUBIC, 7), ((2.0, -1.5, 0.5), 3)])
def test_gram_space_equals_standard(shape, coeffs, steps):
    # the reformulation is exact: X_k = Q_k X0 in exact arithmetic
    rng = np.random.default_rng([7, int(np.prod(shape)), len(shape), shape[0], steps])
    g = rng.standard_normal(shape)
    got = ns.newton_schulz_gram(g, steps, *coeffs, EPS)
    want = ns.newton_schulz(g, steps, *coeffs, EPS)
    assert got.shape == g.shape
    assert np.max(np.abs(got - want)) < 1e-11


@pytest.mark.parametrize("ridge", [0.0, 1e-3, 0.25])
def test_gram_space_ridge_scalar_closed_form(ridge):
    # rows of X0 orthogonal with equal norms: G = s^2 I, so with the ridge the
    # iteration sees g = s^2 (1 + ridge) and Q_k = q_k I with
    # q_{k+1} = q_k (a + b g q_k^2 + c g^2 q_k^4); the result is q_k X0.
    m, n, steps = 6, 15, 5
    rng = np.random.default_rng(3)
    u, _ = np.linalg.qr(rng.standard_normal((n, m)))
    g0 = 2.5 * u.T                           # m x n, orthogonal rows of norm 2.5
    x0 = g0 / (np.sqrt(np.sum(g0 * g0)) + EPS)
    s2 = float(np.sum(x0 * x0)) / m
    gg = s2 * (1.0 + ridge)
    q = 1.0
    for _ in range(steps):
        q = q * (A + B * gg * q * q + C * gg * gg * q ** 4)
    got = ns.newton_schulz_gram(g0, steps, A, B, C, EPS, ridge=ridge)
    assert np.max(np.abs(got - q * x0)) < 1e-12
    # and its transpose goes through the tall path to the same numbers
    got_t = ns.newton_schulz_gram(np.ascontiguousarray(g0.T), steps, A, B, C, EPS, ridge=ridge)
    assert np.max(np.abs(got_t - (q * x0).T)) < 1e-12
