"""Oracle Newton-Schulz: the quintic iteration in float64.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

owner_planning page, ``ns_cost_fn``: view the tensor as (rows, cols) =
(shape[0], product of shape[1:]); normalise it; work on its transpose if rows
> cols so that rows <= cols; then each step is
    A = X X^T,   X = a X + (b A + c A A) X
with scalar coefficients (a, b, c).

Readings taken where the page is silent (each also listed with its reason in
the design notes):
  * the normalisation is by the Frobenius norm plus a small epsilon:
    X0 = X / (||X||_F + eps), so the largest singular value of X0 is <= 1 and a
    zero matrix stays zero;
  * the result is transposed back, so the output has the input's shape;
  * the number of steps defaults to five (``assign_owner_work``'s default
    cost is Newton-Schulz with five iterations).

Pinned by (tests/test_oracle_ns.py): the SVD closed form X_k = U p^k(S) V^T
with p(s) = a s + b s^3 + c s^5; rank-1 and orthonormal-rows special cases;
tall == transpose of wide; zero in, zero out; the cubic (1.5, -0.5, 0)
converging to the polar factor U V^T; singular values bounded by max p on
[0, 1].
"""

from __future__ import annotations

import numpy as np


def bf16_bits_to_f64(bits) -> np.ndarray:
    """Exact value of bf16 bit patterns (uint16), as float64.

    A bf16 value is the top 16 bits of an IEEE binary32 value.
    Pinned by: hand bit patterns in tests/test_oracle_ns.py.
    """
    u = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def newton_schulz(g, steps: int, a: float, b: float, c: float, eps: float) -> np.ndarray:
    """Newton-Schulz orthogonalisation of one tensor, in float64.

    g: array of any shape with ndim >= 2 (values already in float64).
    Returns a float64 array of g's shape.
    """
    g = np.asarray(g, dtype=np.float64)
    if g.ndim < 2:
        raise ValueError("Newton-Schulz needs a tensor with at least 2 dims")
    shape = g.shape
    x = g.reshape(shape[0], -1)
    transposed = x.shape[0] > x.shape[1]
    if transposed:
        x = x.T
    x = x / (np.sqrt(np.sum(x * x)) + eps)
    for _ in range(steps):
        A = x @ x.T
        B = b * A + c * (A @ A)
        x = a * x + B @ x
    if transposed:
        x = x.T
    return np.ascontiguousarray(x).reshape(shape)


def newton_schulz_gram(g, steps: int, a: float, b: float, c: float, eps: float,
                       ridge: float = 0.0) -> np.ndarray:
    """Newton-Schulz evaluated in the m x m Gram space, in float64.

    "[GTP][Muon] Optimize Muon step performance" page, "Secondary (parked)",
    gram_once: an exact Gram-space reformulation of the iteration, hardened
    with an fp32 Gram and a trace ridge. With X0 the normalised (and, if tall,
    transposed) input, every iterate is X_k = Q_k X0 for an m x m matrix Q_k
    (Q_0 = I), so X_k X_k^T = Q_k G Q_k^T with the Gram G = X0 X0^T, computed
    once. Each step is then
        A = Q G Q^T,   Q = a Q + (b A + c A A) Q
    and the result is Q_k X0. Reading taken for the ridge, which the page
    names but does not define: G is replaced by G + ridge (tr(G) / m) I before
    the iteration; ridge = 0 is the exact reformulation.

    Pinned by (tests/test_oracle_ns.py): equality with ``newton_schulz`` for
    ridge = 0, and a scalar closed form for Gram matrices that are multiples of
    the identity (with and without ridge).
    """
    g = np.asarray(g, dtype=np.float64)
    if g.ndim < 2:
        raise ValueError("Newton-Schulz needs a tensor with at least 2 dims")
    shape = g.shape
    x = g.reshape(shape[0], -1)
    transposed = x.shape[0] > x.shape[1]
    if transposed:
        x = x.T
    x0 = x / (np.sqrt(np.sum(x * x)) + eps)
    m = x0.shape[0]
    G = x0 @ x0.T
    if ridge:
        G = G + ridge * (np.trace(G) / m) * np.eye(m)
    Q = np.eye(m)
    for _ in range(steps):
        A = Q @ G @ Q.T
        Q = a * Q + (b * A + c * (A @ A)) @ Q
    out = Q @ x0
    if transposed:
        out = out.T
    return np.ascontiguousarray(out).reshape(shape)
