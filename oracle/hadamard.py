"""The fixed orthonormal 128-wide Hadamard basis (oracle; test infrastructure only).

Cited: "H3 Streamed Blocks" node page, Inputs table, kv_store row, and the
"Low VRAM, low RAM" page, "The K/V store options", rotation paragraph.  Both
call for one fixed orthonormal Hadamard rotation of width 128 over the head
dimension, and neither says how the matrix is built, ordered or signed.  The
reading taken here: Sylvester's doubling construction in natural order, no
sign flips, scaled by 1/sqrt(128).
"""
from __future__ import annotations

import numpy as np


def sylvester_hadamard(n: int = 128) -> np.ndarray:
    """Integer +-1 Hadamard matrix of order n (a power of two) by Sylvester doubling.

    H_1 = [1];  H_2m = [[H_m, H_m], [H_m, -H_m]].
    """
    if n < 1 or n & (n - 1):
        raise ValueError("order must be a power of two")
    h = np.ones((1, 1), dtype=np.int64)
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    return h


def orthonormal_hadamard(n: int = 128) -> np.ndarray:
    """fp64 orthonormal basis H / sqrt(n); symmetric, so it is its own inverse."""
    return sylvester_hadamard(n).astype(np.float64) / np.sqrt(float(n))
