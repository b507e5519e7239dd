"""Test helpers: move seeded inputs between NumPy and torch and run the oracle.

bf16 data travels as uint16 bit patterns on the host, so the oracle sees
exactly the values the GPU sees.
"""

from __future__ import annotations

import sys

import numpy as np


def log(msg: str) -> None:
    """Name the case before each GPU step (flushed, so a hard failure still shows it)."""
    print(msg, file=sys.stderr, flush=True)


def to_device(arr: np.ndarray, dtype: str):
    import torch
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(arr, dtype=np.uint16).view(np.int16))
        return t.view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).cuda()


def to_host(t, dtype: str) -> np.ndarray:
    import torch
    t = t.detach().cpu().contiguous()
    if dtype == "bf16":
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def host_to_f64(arr: np.ndarray, dtype: str) -> np.ndarray:
    from oracle import ns
    if dtype == "bf16":
        return ns.bf16_bits_to_f64(arr)
    return np.asarray(arr, dtype=np.float32).astype(np.float64)


def oracle_ns(arr: np.ndarray, dtype: str, steps: int, coeffs, eps: float) -> np.ndarray:
    """fp64 oracle on the exact input values, with the fp32-rounded coefficients the GPU gets."""
    from oracle import ns
    a, b, c = (float(np.float32(x)) for x in coeffs)
    return ns.newton_schulz(host_to_f64(arr, dtype), steps, a, b, c, float(np.float32(eps)))


# Tolerances (max abs error against the fp64 oracle), fixed for the method's
# workloads: bf16 storage of X, A, B with fp32 accumulation, and all-fp32.
TOL = {"bf16": 2e-2, "f32": 1e-4}
