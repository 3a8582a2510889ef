"""Exact decoding of bf16 / fp16 bit patterns and fp16 rounding (oracle; test infrastructure only)."""
from __future__ import annotations

import numpy as np

FP16_MAX = 65504.0


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Decode bf16 bit patterns (uint16) exactly to float64."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def f16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Decode IEEE binary16 bit patterns (uint16) exactly to float64."""
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def f64_to_f16_bits(x: np.ndarray, saturate: bool = True) -> np.ndarray:
    """Round float64 to IEEE binary16 (nearest, ties to even) and return the bits.

    NumPy's float64 -> float16 cast rounds once and correctly; a test pins it
    against a brute-force nearest search over the fp16 grid.  With ``saturate``
    a finite value beyond the fp16 range maps to +-65504 instead of +-inf.
    """
    x = np.asarray(x, dtype=np.float64)
    if saturate:
        x = np.clip(x, -FP16_MAX, FP16_MAX)
    return x.astype(np.float16).view(np.uint16)
