"""Attention over one head in fp64 (oracle; test infrastructure only).

* exact store: the plain definition O = softmax(Q K^T * scale) V ("H3 Streamed
  Blocks" node page, Inputs table, kv_store row: "bf16 (exact)" is stock math,
  chunked).  Full (non-causal) attention, as in a DiT block.
* kvi8r store: Q is rotated into the Hadamard basis, attends the dequantised
  rotated K/V, and the output is rotated back once (same row; "Low VRAM, low
  RAM" page, "The K/V store options", rotation paragraph).
* tile mask: 64Q x 64KV keep/drop; dropped tiles are excluded from the softmax
  (the hard arm on the "H3-Optimizations" page, Nodes).  A row with nothing kept
  has no defined softmax; the reading taken here is an all-zero output.
* blockwise twin: the same result reached as query chunks x KV blocks with an
  explicit log-sum-exp combine ("H3 Streamed Blocks" node page, Inputs table,
  kv_block and q_chunk rows).  It exists to pin the plain definition.
"""
from __future__ import annotations

import numpy as np

from .encodings import bf16_to_f64
from .hadamard import orthonormal_hadamard
from .kvi8r import dequantize_rows, dequantize_rows_grouped

TILE = 64


def expand_tile_mask(mask_head: np.ndarray, q_rows: np.ndarray, n_kv: int, tile: int = TILE) -> np.ndarray:
    """Boolean keep matrix [len(q_rows), n_kv] from one head's tile mask [nQt, nKt]."""
    q_rows = np.asarray(q_rows)
    return np.asarray(mask_head)[q_rows // tile][:, np.arange(n_kv) // tile] != 0


def attention(q, k, v, scale: float, keep=None, row_block: int = 128) -> np.ndarray:
    """softmax(q k^T * scale) v, row by row, in fp64; keep (bool [n, m]) drops entries."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    out = np.zeros((q.shape[0], v.shape[1]), dtype=np.float64)
    if k.shape[0] == 0:
        return out
    for r0 in range(0, q.shape[0], row_block):
        r1 = min(r0 + row_block, q.shape[0])
        s = (q[r0:r1] @ k.T) * scale
        if keep is not None:
            s = np.where(keep[r0:r1], s, -np.inf)
        m = s.max(axis=1, keepdims=True)
        empty = ~np.isfinite(m)
        p = np.exp(s - np.where(empty, 0.0, m))
        l = p.sum(axis=1, keepdims=True)
        o = (p @ v) / np.where(l == 0.0, 1.0, l)
        out[r0:r1] = np.where(empty, 0.0, o)
    return out


def attention_blockwise(q, k, v, scale: float, q_chunk: int, kv_block: int, keep=None) -> np.ndarray:
    """Same result as ``attention``, computed per query chunk and per KV block.

    Each block b yields (O_b, lse_b) with lse_b = m_b + log sum exp(S - m_b);
    the blocks are merged by O = sum_b exp(lse_b - lse) O_b, lse = log sum_b exp(lse_b).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n, m = q.shape[0], k.shape[0]
    out = np.zeros((n, v.shape[1]), dtype=np.float64)
    for c0 in range(0, n, q_chunk):
        c1 = min(c0 + q_chunk, n)
        outs, lses = [], []
        for b0 in range(0, m, kv_block):
            b1 = min(b0 + kv_block, m)
            s = (q[c0:c1] @ k[b0:b1].T) * scale
            if keep is not None:
                s = np.where(keep[c0:c1, b0:b1], s, -np.inf)
            mb = s.max(axis=1, keepdims=True)
            empty = ~np.isfinite(mb)
            p = np.exp(s - np.where(empty, 0.0, mb))
            lb = p.sum(axis=1, keepdims=True)
            ob = (p @ v[b0:b1]) / np.where(lb == 0.0, 1.0, lb)
            with np.errstate(divide="ignore"):
                lse_b = np.where(empty, -np.inf, mb + np.log(np.where(lb == 0.0, 1.0, lb)))
            outs.append(np.where(empty, 0.0, ob))
            lses.append(lse_b)
        if not lses:
            continue
        lse_all = np.concatenate(lses, axis=1)
        top = lse_all.max(axis=1, keepdims=True)
        none = ~np.isfinite(top)
        top = np.where(none, 0.0, top)
        lse = top + np.log(np.exp(lse_all - top).sum(axis=1, keepdims=True) + none)
        acc = np.zeros((c1 - c0, v.shape[1]), dtype=np.float64)
        for ob, lse_b in zip(outs, lses):
            acc += np.exp(lse_b - lse) * ob
        out[c0:c1] = np.where(none, 0.0, acc)
    return out


def exact_attention_bf16(q_bits, k_bits, v_bits, scale: float, keep=None) -> np.ndarray:
    """Exact-store attention of one head from bf16 bit patterns [n,128], [m,128], [m,128]."""
    return attention(bf16_to_f64(q_bits), bf16_to_f64(k_bits), bf16_to_f64(v_bits), scale, keep)


def kvi8r_attention(q, k_codes, k_scale_bits, v_codes, v_scale_bits, scale: float, keep=None) -> np.ndarray:
    """kvi8r attention of one head.

    q: fp64 [n, 128] in the original basis.  K/V: int8 codes [m, 128] and fp16
    scale bits in the rotated basis, [m] (one per row) or [m, 4] (one per 32
    values, the per-32-value variant).  q' = q H; O' = softmax(q' K^T s) V with
    K, V the exact dequantised rows; O = O' H^T (= O' H, H symmetric).
    """
    h = orthonormal_hadamard(np.asarray(q).shape[-1])
    q_rot = np.asarray(q, dtype=np.float64) @ h
    o_rot = attention(q_rot, _dequantize(k_codes, k_scale_bits), _dequantize(v_codes, v_scale_bits), scale, keep)
    return o_rot @ h.T


def _dequantize(codes, scale_bits):
    if np.asarray(scale_bits).ndim == 2:
        return dequantize_rows_grouped(codes, scale_bits)
    return dequantize_rows(codes, scale_bits)
