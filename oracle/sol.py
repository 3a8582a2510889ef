"""Tile-masked attention with a residual for the dropped tiles (oracle; test infrastructure only).

Cited: "H3-Optimizations" page, Nodes, routed-geometry paragraph.  Two arms
are described there: the hard arm leaves rejected 64Q x 64KV tiles out of the
softmax; the Sol arm keeps a summary of each rejected tile (the mean of its
keys, the sum of its values) and folds that into the online-softmax state.  No
formula is given; the reading taken here:

* a dropped KV tile t with n_t keys (64, or fewer for the last tile of the
  store) becomes one pseudo-key: k_t = mean of its keys, value v_t = mean of its
  values (block sum / n_t), counted n_t times;
* its softmax weight is therefore n_t * exp(q . k_t * scale), and it adds that
  weight times v_t to the numerator: exp(q . k_t * scale) times the block sum
  of V, as the page's block-sum V suggests;
* kept tiles contribute their keys exactly, as in the hard arm.

When the keys of a dropped tile are all equal, the pseudo-key reproduces the
tile exactly; the tests pin the residual on that closed form.  Plain fp64
NumPy, per query tile.
"""
from __future__ import annotations

import numpy as np

from .encodings import bf16_to_f64
from .hadamard import orthonormal_hadamard
from .kvi8r import dequantize_rows, dequantize_rows_grouped

TILE = 64


def tile_summaries(k, v, tile: int = TILE):
    """Per KV tile: mean key, mean value and key count (fp64)."""
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    m = k.shape[0]
    nt = (m + tile - 1) // tile
    kbar = np.zeros((nt, k.shape[1]))
    vbar = np.zeros((nt, v.shape[1]))
    count = np.zeros(nt)
    for t in range(nt):
        r0, r1 = t * tile, min((t + 1) * tile, m)
        kbar[t] = k[r0:r1].mean(axis=0)
        vbar[t] = v[r0:r1].mean(axis=0)
        count[t] = r1 - r0
    return kbar, vbar, count


def sol_attention(q, k, v, scale: float, q_rows, mask_head, tile: int = TILE) -> np.ndarray:
    """Attention of query rows q (global indices q_rows) over the kept keys of their
    q-tile plus one pseudo-key per dropped tile (mean K, mean V, weight n_t)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    q_rows = np.asarray(q_rows)
    mask_head = np.asarray(mask_head)
    m = k.shape[0]
    kbar, vbar, count = tile_summaries(k, v, tile)
    tile_of_key = np.arange(m) // tile
    out = np.zeros((q.shape[0], v.shape[1]))
    for qt in np.unique(q_rows // tile):
        sel = np.nonzero(q_rows // tile == qt)[0]
        keep_t = mask_head[qt] != 0
        kept = keep_t[tile_of_key]
        drop = np.nonzero(~keep_t)[0]
        keys = np.concatenate([k[kept], kbar[drop]])
        vals = np.concatenate([v[kept], vbar[drop]])
        log_w = np.concatenate([np.zeros(int(kept.sum())), np.log(count[drop])])
        if keys.shape[0] == 0:
            continue
        s = (q[sel] @ keys.T) * scale + log_w
        mx = s.max(axis=1, keepdims=True)
        p = np.exp(s - mx)
        out[sel] = (p @ vals) / p.sum(axis=1, keepdims=True)
    return out


def exact_sol_attention_bf16(q_bits, k_bits, v_bits, scale: float, q_rows, mask_head) -> np.ndarray:
    """Exact store: bf16 bit patterns of one head."""
    return sol_attention(bf16_to_f64(q_bits), bf16_to_f64(k_bits), bf16_to_f64(v_bits), scale, q_rows, mask_head)


def kvi8r_sol_attention(q, k_codes, k_scale_bits, v_codes, v_scale_bits, scale: float, q_rows,
                        mask_head) -> np.ndarray:
    """kvi8r store (scales [m] per row or [m, 4] per 32 values): tile summaries of the dequantised
    rotated K/V; q rotated in, O rotated back."""
    h = orthonormal_hadamard(np.asarray(q).shape[-1])
    q_rot = np.asarray(q, dtype=np.float64) @ h
    deq = dequantize_rows_grouped if np.asarray(k_scale_bits).ndim == 2 else dequantize_rows
    o_rot = sol_attention(q_rot, deq(k_codes, k_scale_bits), deq(v_codes, v_scale_bits), scale, q_rows, mask_head)
    return o_rot @ h.T
