"""Per-row routing between the exact store and the kvi8r store (oracle; test infrastructure only).

"H3 Streamed Blocks (exact low-VRAM, alpha)" node page, Inputs table,
exact_av_rows row: the text and audio query rows are sent through exact bf16
attention over a K/V kept in bf16, while the video rows stay on the quantised
store.  The page ties the switch to its fp4 store; the routing itself carries
over to kvi8r unchanged.  Reading taken here: the routed rows are given as
[begin, end) spans of query rows (text and audio are contiguous stretches of
the packed sequence); a row inside a span gets exact attention over the bf16
K/V, every other row kvi8r attention over the store.  Both stores hold the same
keys and values.  Plain fp64 NumPy.
"""
from __future__ import annotations

import numpy as np

from .attention import exact_attention_bf16, kvi8r_attention
from .encodings import bf16_to_f64


def spans_to_rows(spans, n_rows: int) -> np.ndarray:
    """Boolean [n_rows]: True for rows inside one of the [begin, end) spans.

    Spans must be increasing, disjoint and inside [0, n_rows]; empty spans
    (begin == end) are allowed.
    """
    rows = np.zeros(n_rows, dtype=bool)
    prev_end = 0
    for begin, end in spans:
        begin, end = int(begin), int(end)
        if not (prev_end <= begin <= end <= n_rows):
            raise ValueError(f"span [{begin}, {end}) out of order or outside [0, {n_rows}]")
        rows[begin:end] = True
        prev_end = end
    return rows


def routed_attention(q_bits, k_bits, v_bits, k_codes, k_scale_bits, v_codes, v_scale_bits, scale: float,
                     exact_rows) -> np.ndarray:
    """One head: rows with exact_rows[i] attend the bf16 K/V exactly, the others the kvi8r store.

    q_bits, k_bits, v_bits: bf16 bit patterns [n,128], [m,128], [m,128];
    k_codes, v_codes: int8 [m,128] and k_scale_bits, v_scale_bits: fp16 bits [m]
    of the kvi8r store built from the same K and V.
    """
    q_bits = np.asarray(q_bits)
    exact_rows = np.asarray(exact_rows, dtype=bool)
    out = np.zeros((q_bits.shape[0], np.asarray(v_bits).shape[1]))
    if exact_rows.any():
        out[exact_rows] = exact_attention_bf16(q_bits[exact_rows], k_bits, v_bits, scale)
    if (~exact_rows).any():
        out[~exact_rows] = kvi8r_attention(bf16_to_f64(q_bits[~exact_rows]), k_codes, k_scale_bits, v_codes,
                                           v_scale_bits, scale)
    return out
