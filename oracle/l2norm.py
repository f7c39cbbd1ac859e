"""fp64 L2 normalisation of query/key rows, the optional normaliser of the
scalar-g kernel page (its in-kernel q/k normalisation): every row x over the
key dimension becomes x * rsqrt(sum(x^2) + 1e-6).

TEST INFRASTRUCTURE ONLY: imported by tests/, never by the product path.
With in-kernel normalisation requested, the oracle's inputs are the raw q, k
passed through this function, then the recurrence.
"""
from __future__ import annotations

import numpy as np

EPS = 1e-6


def l2norm_rows(x) -> np.ndarray:
    """Normalise the last axis of x in fp64: x / sqrt(sum_d x_d^2 + 1e-6)."""
    x = np.asarray(x, dtype=np.float64)
    out = np.empty_like(x)
    flat_in = x.reshape(-1, x.shape[-1])
    flat_out = out.reshape(-1, x.shape[-1])
    for i in range(flat_in.shape[0]):
        row = flat_in[i]
        flat_out[i] = row / np.sqrt(np.dot(row, row) + EPS)
    return out
