"""Seeded synthetic inputs shared by the tests, the bench and the oracle checks.

This module only *draws* inputs: Gaussian Q/K/V rows rounded to bf16 bit
patterns, the seeded outlier channels of K, the seeded 64x64 tile mask and the
seeded sample of query rows.  It holds none of the method's arithmetic (no
rotation, no quantisation, no attention).

Workload shapes follow the pages: a packed DiT sequence of about 217k tokens
("H3 Streamed Blocks" node page, intro; "Low VRAM, low RAM" page, "The numbers"),
head dim 128 and chunk defaults of 16384 ("H3 Streamed Blocks" node page,
Inputs table: q_chunk, kv_chunk, kv_block and kv_store rows), and 64Q x 64KV tile
routing at a 30 % video-KV budget with the text prefix kept dense
("H3-Optimizations" page, Nodes: H3 Sparse Attention and its Advanced variant).

Random streams: every (tensor, head) pair has its own PCG64 stream seeded with
SeedSequence([seed, stream, head]) so any single head can be regenerated alone.
Streams: 0 = Q, 1 = K, 2 = V, 3 = outlier channels of K, 4 = tile mask,
5 = sampled query rows, 6 = sampled video query tiles.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

HEAD_DIM = 128
TILE = 64

STREAM_Q, STREAM_K, STREAM_V, STREAM_OUTLIER, STREAM_MASK, STREAM_ROWS, STREAM_QTILES = 0, 1, 2, 3, 4, 5, 6


@dataclass(frozen=True)
class Workload:
    """One synthetic workload: shapes, seed, input structure and chunking."""

    name: str
    seq: int
    heads: int
    seed: int
    q_chunk: int
    kv_block: int
    k_outliers: bool = False
    sparse: bool = False
    text_prefix: int = 0          # tokens of dense text prefix (sparse workloads)
    video_kv_density: float = 0.0  # fraction of video KV tiles kept per video q-tile
    oracle_rows_per_head: int = 0  # 0 = every row
    extra: dict = field(default_factory=dict)

    @property
    def n_tiles(self) -> int:
        return (self.seq + TILE - 1) // TILE


# The five workloads.  tiny: all rows checked in seconds.  outlier16k / outlier64k:
# K carries 4 seeded outlier channels per head scaled x20 before bf16 rounding.
# long217k: the long de-rope pass length.  sparse64k: outlier64k's tensors with a
# 512-token dense text prefix and 305 of 1016 video KV tiles kept per video q-tile.
WORKLOADS = {
    "tiny": Workload("tiny", 1024, 2, 1, 256, 256),
    "outlier16k": Workload("outlier16k", 16384, 8, 2, 4096, 4096, k_outliers=True),
    "outlier64k": Workload("outlier64k", 65536, 32, 3, 16384, 16384, k_outliers=True,
                           oracle_rows_per_head=2048),
    "long217k": Workload("long217k", 217088, 32, 4, 16384, 16384, oracle_rows_per_head=2048),
    "sparse64k": Workload("sparse64k", 65536, 32, 3, 16384, 16384, k_outliers=True,
                          sparse=True, text_prefix=512, video_kv_density=0.30,
                          oracle_rows_per_head=2048),
}


def _rng(seed: int, stream: int, head: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, stream, head])))


def bf16_bits_from_f32(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even); return the bit patterns."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def _round_bf16_into(buf: np.ndarray, tmp: np.ndarray, dest: np.ndarray) -> None:
    """Same rounding as bf16_bits_from_f32, in place on reusable buffers (buf is clobbered)."""
    u = buf.view(np.uint32)
    np.right_shift(u, np.uint32(16), out=tmp)
    tmp &= np.uint32(1)
    tmp += np.uint32(0x7FFF)
    u += tmp
    u >>= np.uint32(16)
    np.copyto(dest, u, casting="unsafe")


def outlier_channels(seed: int, head: int, count: int = 4) -> np.ndarray:
    """The seeded distinct outlier channels of K for one head."""
    return np.sort(_rng(seed, STREAM_OUTLIER, head).choice(HEAD_DIM, size=count, replace=False))


def _draw(w: Workload, tensor: str, head: int, out: np.ndarray) -> np.ndarray:
    stream = {"q": STREAM_Q, "k": STREAM_K, "v": STREAM_V}[tensor]
    _rng(w.seed, stream, head).standard_normal(out=out, dtype=np.float32)
    if tensor == "k" and w.k_outliers:
        out[:, outlier_channels(w.seed, head)] *= np.float32(20.0)
    return out


def head_rows_f32(w: Workload, tensor: str, head: int) -> np.ndarray:
    """float32 [S, 128] draws for one (tensor, head) before bf16 rounding."""
    return _draw(w, tensor, head, np.empty((w.seq, HEAD_DIM), dtype=np.float32))


def head_bf16(w: Workload, tensor: str, head: int) -> np.ndarray:
    """bf16 bit patterns [S, 128] of one (tensor, head)."""
    return bf16_bits_from_f32(head_rows_f32(w, tensor, head))


def _workers() -> int:
    n = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    return max(1, min(16, n))


def for_each_head(w: Workload, tensors, sink, workers: int | None = None) -> None:
    """Call sink(tensor, head, bits) for every (tensor, head), bits = uint16 [S, 128].

    Draws run in a thread pool with per-thread reusable buffers; ``bits`` is
    only valid during the call (copy it if it must outlive the call).
    """
    import threading

    local = threading.local()

    def job(th):
        t, h = th
        if not hasattr(local, "f"):
            local.f = np.empty((w.seq, HEAD_DIM), dtype=np.float32)
            local.tmp = np.empty((w.seq, HEAD_DIM), dtype=np.uint32)
            local.bits = np.empty((w.seq, HEAD_DIM), dtype=np.uint16)
        _draw(w, t, h, local.f)
        _round_bf16_into(local.f, local.tmp, local.bits)
        sink(t, h, local.bits)

    jobs = [(t, h) for t in tensors for h in range(w.heads)]
    with ThreadPoolExecutor(workers or _workers()) as ex:
        list(ex.map(job, jobs))


def qkv_bf16(w: Workload, tensors=("q", "k", "v")) -> dict:
    """Token-major bf16 bit patterns [S, H, 128] (uint16) for the requested tensors."""
    out = {t: np.empty((w.seq, w.heads, HEAD_DIM), dtype=np.uint16) for t in tensors}

    def sink(t, h, bits):
        out[t][:, h, :] = bits

    for_each_head(w, tensors, sink)
    return out


def sampled_rows(w: Workload, head: int, n: int | None = None) -> np.ndarray:
    """Sorted seeded sample of query rows of one head (all rows when n covers S)."""
    n = w.oracle_rows_per_head if n is None else n
    if n <= 0 or n >= w.seq:
        return np.arange(w.seq)
    return np.sort(_rng(w.seed, STREAM_ROWS, head).choice(w.seq, size=n, replace=False))


def tile_mask(w: Workload) -> np.ndarray:
    """uint8 keep mask [H, nQt, nKt] at 64Q x 64KV granularity.

    Query tiles inside the text prefix keep every KV tile.  Every other query
    tile keeps all prefix KV tiles plus exactly round(density * n_video) video KV
    tiles drawn without replacement from that (head, q-tile)'s seeded stream.
    """
    nt = w.n_tiles
    text = (w.text_prefix + TILE - 1) // TILE
    n_video = nt - text
    keep = int(round(w.video_kv_density * n_video))
    mask = np.zeros((w.heads, nt, nt), dtype=np.uint8)
    for h in range(w.heads):
        rng = _rng(w.seed, STREAM_MASK, h)
        mask[h, :text, :] = 1
        mask[h, text:, :text] = 1
        for qt in range(text, nt):
            mask[h, qt, text + rng.choice(n_video, size=keep, replace=False)] = 1
    return mask


def sampled_q_tiles(w: Workload, head: int, n_video: int = 24) -> np.ndarray:
    """Sorted 64-row query tiles of one head for an oracle sample of a tile-masked workload: every
    text-prefix tile plus n_video video tiles drawn without replacement from the head's stream."""
    text = (w.text_prefix + TILE - 1) // TILE
    n_vid = w.n_tiles - text
    video = text + _rng(w.seed, STREAM_QTILES, head).choice(n_vid, size=min(n_video, n_vid), replace=False)
    return np.sort(np.concatenate([np.arange(text), video]))


def q_tile_rows(w: Workload, tiles: np.ndarray) -> np.ndarray:
    """Query rows of the given 64-row tiles, clipped to the sequence."""
    rows = (np.asarray(tiles)[:, None] * TILE + np.arange(TILE)[None, :]).reshape(-1)
    return rows[rows < w.seq]
