"""kvi8r quantisation of K/V rows (oracle; test infrastructure only).

Follows the "H3 Streamed Blocks" node page, Inputs table, kv_store row, and the
"Low VRAM, low RAM" page, "The K/V store options" (the kvi8r row of the store
table and the rotation paragraph): each (token, head) row of 128 values goes
into the fixed orthonormal Hadamard basis and is kept as int8 codes with one
fp16 scale.

Readings where the pages are silent (each is listed in the design notes):

* grid: symmetric, no zero point, scale = absmax / 127, codes clamped to
  [-127, 127] (never -128);
* the codes are taken against the *stored* (fp16-rounded) scale, so every
  element keeps |y - q*s| <= s/2 and the absmax element gets |q| = 127;
* the scale is the fp64 value absmax/127 rounded once to fp16 (nearest, ties
  to even); a zero row gets scale 0 and all-zero codes; a row whose scale
  would overflow fp16 saturates to 65504 and its codes clamp;
* the code is the definition itself, q = clip(rint(y / s)) on fp64 y and the
  fp64 value of the stored scale, rounding half to even.

A code is an integer chosen by floating point, so an implementation that
evaluates y / s in lower precision can land on the other side of a
half-integer when y / s sits very close to one.  ``fp32_decision_width`` bounds
that distance for an evaluation in fp32 (butterflies, then one product with an
fp32 reciprocal of the scale), and ``near_ties`` flags the elements inside the
band.  Outside the band only the code above is correct; inside it both
neighbours are.

Per-32-value variant ("Low VRAM, low RAM" page, "What is next": a kvi8r variant
with one scale for every 32 values, finer than one per row).  Reading: each
rotated row is cut into four groups of 32 consecutive values (rotated dims
0-31, 32-63, 64-95, 96-127) and every group is quantised exactly as a row is
above, with its own fp16 scale.
"""
from __future__ import annotations

import numpy as np

from .encodings import f16_to_f64, f64_to_f16_bits
from .hadamard import orthonormal_hadamard

QMAX = 127
GROUP = 32  # values per scale in the per-32-value variant
FP32_UNIT = 2.0 ** -24  # unit roundoff of binary32
FP64_UNIT = 2.0 ** -53  # unit roundoff of binary64


def rotate_rows(x: np.ndarray) -> np.ndarray:
    """y = x H for row vectors x [n, 128], with H the orthonormal Hadamard basis (fp64)."""
    x = np.asarray(x, dtype=np.float64)
    return x @ orthonormal_hadamard(x.shape[-1])


def row_scales(y: np.ndarray) -> np.ndarray:
    """fp16 bit patterns of the per-row scale absmax(y)/127."""
    a = np.abs(np.asarray(y, dtype=np.float64)).max(axis=-1)
    return f64_to_f16_bits(a / QMAX, saturate=True)


def _code_variable(y: np.ndarray, scale_bits: np.ndarray):
    """(y / s in fp64, zero-scale mask) for rows y [n, k] and scales [n]."""
    s = f16_to_f64(scale_bits)
    zero = s == 0
    with np.errstate(divide="ignore", invalid="ignore"):
        v = np.asarray(y, dtype=np.float64) / np.where(zero, 1.0, s)[:, None]
    v[zero] = 0.0
    return v, zero


def codes_for_scales(y: np.ndarray, scale_bits: np.ndarray) -> np.ndarray:
    """int8 codes of rotated rows y [n, k] against given fp16 scales [n].

    q = clip(rint(y / s), -127, 127) with y and s in fp64 (rint rounds half to
    even).  A zero scale gives zero codes.
    """
    v, _ = _code_variable(y, scale_bits)
    return np.clip(np.rint(v), -QMAX, QMAX).astype(np.int8)


def fp32_decision_width(x: np.ndarray, scale_bits: np.ndarray, group: int = 128) -> np.ndarray:
    """Per-element bound on |v' - y/s| when the code variable v' is evaluated in fp32.

    The evaluation bounded here: the unnormalised transform z = x H sqrt(128)
    by seven radix-2 butterfly stages in fp32 on the exact (bf16) inputs, then
    v' = z' * r' with r' = fp32(1 / (s sqrt(128))), the product exact (one
    fused multiply-add rounds it straight to an integer).  Standard error
    analysis of a depth-7 summation tree gives |z' - z| <= g7 * sum|x| with
    g7 = 7u / (1 - 7u), u = 2^-24, and |r' - r| <= u r, so

        |v' - v| <= g7 (1 + u) r sum|x| + u |v|.

    The oracle's own fp64 evaluation of y and y / s adds at most
    (130 u64 r sum|x| + 2 u64 |v|), u64 = 2^-53, which is added too.
    x: the row's 128 decoded inputs [n, 128]; scale_bits: [n] (one scale per
    row) or [n, 128 // group] (one per group).  Returns [n, 128].
    """
    x = np.asarray(x, dtype=np.float64)
    n, d = x.shape
    s = f16_to_f64(scale_bits).reshape(n, -1)
    ng = s.shape[1]
    if ng * group != d and ng != 1:
        raise ValueError("scale_bits must hold one scale per row or one per group")
    s = np.repeat(s, d // ng, axis=1)
    sum_abs = np.abs(x).sum(axis=1, keepdims=True)
    y = rotate_rows(x)
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.where(s > 0, 1.0 / (s * np.sqrt(float(d))), 0.0)
        v = np.where(s > 0, y / np.where(s > 0, s, 1.0), 0.0)
    g7 = 7 * FP32_UNIT / (1 - 7 * FP32_UNIT)
    return (g7 * (1 + FP32_UNIT) + 130 * FP64_UNIT) * r * sum_abs + (FP32_UNIT + 2 * FP64_UNIT) * np.abs(v)


def near_ties(y: np.ndarray, scale_bits: np.ndarray, width: np.ndarray) -> np.ndarray:
    """True where y / s lies within ``width`` of a half-integer (k + 1/2).

    There, the code is settled by the rounding error of the evaluation and both
    neighbours k and k + 1 are correct codes.  Rows with a zero scale have no ties.
    y: [n, k]; scale_bits: [n]; width: broadcastable to y.
    """
    v, zero = _code_variable(y, scale_bits)
    dist = np.abs(v - (np.floor(v) + 0.5))
    out = dist <= width
    out[zero] = False
    return out


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
