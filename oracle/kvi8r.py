"""kvi8r quantisation of K/V rows (oracle; test infrastructure only).

Follows "H3 Streamed Blocks" node page, Inputs table, kv_store row, and "Low
VRAM, low RAM" page, "The K/V store options" (table row for kvi8r and the
rotation paragraph): each (token, head) row of 128 values is rotated into the
fixed orthonormal Hadamard basis and stored as int8 codes with one fp16 scale.

Readings where the pages are silent (each is listed in the design notes):

* grid: symmetric, no zero point, scale = absmax / 127, codes clamped to
  [-127, 127] (never -128);
* the codes are taken against the *stored* (fp16-rounded) scale, so every
  element keeps |y - q*s| <= s/2 and the absmax element gets |q| = 127;
* the scale is the fp64 value absmax/127 rounded once to fp16 (nearest, ties
  to even); a zero row gets scale 0 and all-zero codes; a row whose scale
  would overflow fp16 saturates to 65504 and its codes clamp;
* the code is an integer decided by floating point, so it is decided in the
  kernel's precision, fp32: q = round-half-even(fp32(y) / fp32(s)) with the
  quotient correctly rounded to fp32.  Every other step is fp64.

Per-32-value variant ("Low VRAM, low RAM" page, "What is next": a kvi8r variant
with a scale per 32 values, finer than per row).  Reading: each rotated row is
cut into four groups of 32 consecutive values (rotated dims 0-31, 32-63, 64-95,
96-127) and every group is quantised exactly as a row is above, with its own
fp16 scale.
"""
from __future__ import annotations

import numpy as np

from .encodings import f16_to_f64, f64_to_f16_bits
from .hadamard import orthonormal_hadamard

QMAX = 127
GROUP = 32  # values per scale in the per-32-value variant


def rotate_rows(x: np.ndarray) -> np.ndarray:
    """y = x H for row vectors x [n, 128], with H the orthonormal Hadamard basis (fp64)."""
    x = np.asarray(x, dtype=np.float64)
    return x @ orthonormal_hadamard(x.shape[-1])


def row_scales(y: np.ndarray) -> np.ndarray:
    """fp16 bit patterns of the per-row scale absmax(y)/127."""
    a = np.abs(np.asarray(y, dtype=np.float64)).max(axis=-1)
    return f64_to_f16_bits(a / QMAX, saturate=True)


def codes_for_scales(y: np.ndarray, scale_bits: np.ndarray) -> np.ndarray:
    """int8 codes of rotated rows y [n, 128] against given fp16 scales [n].

    The decision is taken in fp32: fp32(y) / fp32(s), correctly rounded, then
    rounded half to even and clamped to [-127, 127].  A zero scale gives zero codes.
    """
    y32 = np.asarray(y, dtype=np.float64).astype(np.float32)
    s32 = f16_to_f64(scale_bits).astype(np.float32)
    zero = s32 == 0
    with np.errstate(divide="ignore", invalid="ignore"):
        v = y32 / np.where(zero, np.float32(1), s32)[:, None]
    q = np.clip(np.rint(v), -QMAX, QMAX)
    q[zero] = 0
    return q.astype(np.int8)


def quantize_rows(x: np.ndarray):
    """Quantise rows x [n, 128] (already-decoded fp64 values).

    Returns (codes int8 [n, 128], scale bits uint16 [n], y fp64 [n, 128]).
    """
    y = rotate_rows(x)
    s = row_scales(y)
    return codes_for_scales(y, s), s, y


def dequantize_rows(codes: np.ndarray, scale_bits: np.ndarray) -> np.ndarray:
    """Rotated-basis rows codes * scale, exact in fp64."""
    return np.asarray(codes, dtype=np.float64) * f16_to_f64(scale_bits)[:, None]


def quantize_rows_grouped(x: np.ndarray, group: int = GROUP):
    """Per-group variant of quantize_rows: every `group` consecutive rotated values get their own scale.

    Returns (codes int8 [n, 128], scale bits uint16 [n, 128 // group], y fp64 [n, 128]).
    """
    y = rotate_rows(x)
    n, d = y.shape
    yg = y.reshape(n * (d // group), group)  # one group per row
    s = row_scales(yg)
    return codes_for_scales(yg, s).reshape(n, d), s.reshape(n, d // group), y


def dequantize_rows_grouped(codes: np.ndarray, scale_bits: np.ndarray) -> np.ndarray:
    """Rotated-basis rows: each code times the scale of its group, exact in fp64."""
    codes = np.asarray(codes, dtype=np.float64)
    n, d = codes.shape
    g = np.asarray(scale_bits).shape[1]
    return (codes.reshape(n, g, d // g) * f16_to_f64(scale_bits)[:, :, None]).reshape(n, d)
