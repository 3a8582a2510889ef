"""GPU parity of the Sol residual (through the C ABI) against the fp64 oracle.

"H3-Optimizations" page, Nodes, routed-geometry paragraph: besides the hard arm,
a Sol arm stands in for every rejected 64Q x 64KV tile with its block-mean K and
block-sum V.  Reading (oracle/sol.py): a dropped tile of n keys is one
pseudo-key (mean key, mean value) of weight n * exp(scale * q . mean key).

Pins of the GPU path independent of the oracle's Sol arm: when every tile's
keys and values are constant, the pseudo-key reproduces its tile exactly, so
Sol attention under any mask equals plain dense attention (oracle); with every
tile kept, Sol equals dense attention bitwise.  Tolerances are those of the
dense path (kvi8r: relative L2 <= 2e-3, max abs <= 1e-2 on the same store;
exact: relative L2 <= 4e-3); the tile means are rounded once to the
matrix-core type, well inside them.
"""
import numpy as np
import pytest
import torch

import oracle
import store_kvi8r_quantize_amd as h3a
import synth
from gpu_common import (EXACT_REL_L2, KVI8R_MAX_ABS, KVI8R_REL_L2, SCALE, build_store, gpu_u16, host_u16, out_f64,
                        out_like, rel_l2, say, store_head)

pytestmark = pytest.mark.gpu


def _run(mode, q, k, v, store, q_chunk, mask, sol=True):
    out = out_like(q, mode)
    if mode == "kvi8r":
        kc, vc, sc = store
        h3a.h3a_attention(q, kc, vc, sc, out, q_chunk=q_chunk, mode="kvi8r", tile_mask=mask, sol=sol)
    else:
        h3a.h3a_attention(q, k, v, None, out, q_chunk=q_chunk, mode="exact", tile_mask=mask, sol=sol)
    torch.cuda.synchronize()
    return out


def _sol_ref(mode, bits_of, store, h, rows, mask_h):
    """Oracle Sol attention of one head's rows; bits_of(t, h) gives host bf16 bits."""
    if mode == "kvi8r":
        kc, ks, vc, vs = store_head(*store, h)
        return oracle.kvi8r_sol_attention(oracle.bf16_to_f64(bits_of("q", h)[rows]), kc, ks, vc, vs, SCALE, rows,
                                          mask_h)
    return oracle.exact_sol_attention_bf16(bits_of("q", h)[rows], bits_of("k", h), bits_of("v", h), SCALE, rows,
                                           mask_h)


def _assert_close(mode, got, ref, tag):
    r = rel_l2(got, ref)
    mx = float(np.abs(got - ref).max())
    say(tag, mode, "relL2", r, "max abs", mx)
    if mode == "kvi8r":
        assert r <= KVI8R_REL_L2 and mx <= KVI8R_MAX_ABS
    else:
        assert r <= EXACT_REL_L2


def _rows_out(out, rows, h):
    return out_f64(out[torch.from_numpy(np.asarray(rows)).cuda(), h])


@pytest.mark.parametrize("mode", ["exact", "kvi8r"])
def test_sol_random_mask_all_rows(mode):
    # 1000 tokens: a ragged last KV tile of 40 keys; q-tile 3 keeps nothing (pseudo-keys only),
    # q-tile 5 keeps everything (no pseudo-keys), the rest keep ~30% of their tiles.
    w = synth.Workload("sol-masked", 1000, 2, 12, 256, 0)
    bits = synth.qkv_bf16(w)
    g = {t: gpu_u16(bits[t]) for t in bits}
    nt = w.n_tiles
    rng = np.random.default_rng(7)
    mask = (rng.random((2, nt, nt)) < 0.3).astype(np.uint8)
    mask[:, 3, :] = 0
    mask[:, 5, :] = 1
    store = build_store(g["k"], g["v"]) if mode == "kvi8r" else None
    m = torch.from_numpy(mask).cuda()
    out = _run(mode, g["q"], g["k"], g["v"], store, 256, m)
    assert bool(out[192:256].abs().float().sum() > 0)  # the all-dropped q-tile attends the pseudo-keys
    rows = np.arange(w.seq)
    got, ref = [], []
    for h in range(w.heads):
        got.append(_rows_out(out, rows, h))
        ref.append(_sol_ref(mode, lambda t, hh: bits[t][:, hh], store, h, rows, mask[h]))
    _assert_close(mode, np.concatenate(got), np.concatenate(ref), "sol-masked")
    # each row depends only on its own q-tile's lists and the store's tile means
    out64 = _run(mode, g["q"], g["k"], g["v"], store, 64, m)
    assert torch.equal(out.view(torch.int16), out64.view(torch.int16))
    # q-tile 5 drops nothing: the hard arm gives the same bits there
    hard = _run(mode, g["q"], g["k"], g["v"], store, 256, m, sol=False)
    assert torch.equal(out[320:384].view(torch.int16), hard[320:384].view(torch.int16))


@pytest.mark.parametrize("mode", ["exact", "kvi8r"])
def test_sol_constant_tiles_equal_dense_attention(mode):
    # Every KV tile's 64 keys (32 in the ragged last one) are one repeated row, likewise
    # its values, so each pseudo-key stands exactly for its tile: Sol under any mask is
    # plain dense attention, checked against the oracle's dense attention.
    s, heads = 4000, 4
    w = synth.Workload("sol-const", s, heads, 21, 1024, 0)
    bits = synth.qkv_bf16(w)
    tile_of = np.arange(s) // 64
    for t in ("k", "v"):
        bits[t] = np.ascontiguousarray(bits[t][tile_of * 64])  # row r takes the first row of its tile
    g = {t: gpu_u16(bits[t]) for t in bits}
    nt = w.n_tiles
    rng = np.random.default_rng(8)
    mask = (rng.random((heads, nt, nt)) < 0.25).astype(np.uint8)
    mask[:, 0, :] = 0
    store = build_store(g["k"], g["v"]) if mode == "kvi8r" else None
    out = _run(mode, g["q"], g["k"], g["v"], store, 1024, torch.from_numpy(mask).cuda())
    rows = np.arange(s)
    got, ref = [], []
    for h in range(heads):
        got.append(_rows_out(out, rows, h))
        if mode == "kvi8r":
            kc, ks, vc, vs = store_head(*store, h)
            ref.append(oracle.kvi8r_attention(oracle.bf16_to_f64(bits["q"][:, h]), kc, ks, vc, vs, SCALE))
        else:
            ref.append(oracle.exact_attention_bf16(bits["q"][:, h], bits["k"][:, h], bits["v"][:, h], SCALE))
    _assert_close(mode, np.concatenate(got), np.concatenate(ref), "sol-const")


@pytest.mark.parametrize("mode", ["exact", "kvi8r"])
def test_sol_all_kept_equals_dense_bitwise(mode):
    w = synth.WORKLOADS["outlier16k"]
    bits = synth.qkv_bf16(w)
    g = {t: gpu_u16(bits[t]) for t in bits}
    store = build_store(g["k"], g["v"]) if mode == "kvi8r" else None
    nt = w.n_tiles
    ones = torch.ones((w.heads, nt, nt), dtype=torch.uint8, device="cuda")
    dense = out_like(g["q"], mode)
    if mode == "kvi8r":
        h3a.h3a_attention(g["q"], *store, dense, q_chunk=4096, mode="kvi8r")
    else:
        h3a.h3a_attention(g["q"], g["k"], g["v"], None, dense, q_chunk=4096, mode="exact")
    sol = _run(mode, g["q"], g["k"], g["v"], store, 4096, ones)
    assert torch.equal(dense.view(torch.int16), sol.view(torch.int16))


@pytest.mark.timeout(900)
@pytest.mark.parametrize("mode", ["kvi8r", "exact"])
def test_sol_sparse64k_oracle_sample(mode, oracle_pool):
    # every text q-tile (8) plus 24 seeded video q-tiles of each of the 32 heads: 2048 rows per head
    from gpu_common import gpu_inputs, pool_check

    w = synth.WORKLOADS["sparse64k"]
    say("generating", w.name)
    g = gpu_inputs(w)
    mask = synth.tile_mask(w)
    store = build_store(g["k"], g["v"], kv_chunk=w.q_chunk) if mode == "kvi8r" else None
    out = _run(mode, g["q"], g["k"], g["v"], store, w.q_chunk, torch.from_numpy(mask).cuda())
    pool_check(oracle_pool, "sol_" + mode, w, out, range(w.heads),
               lambda h: synth.q_tile_rows(w, synth.sampled_q_tiles(w, h)), store, mask=mask, tag="sol-sparse64k")


@pytest.mark.parametrize("mode", ["exact", "kvi8r"])
def test_sol_single_short_tile(mode):
    # s_kv = 40: one KV tile of 40 keys.  q-tile 0 drops it, so its only key is the pseudo-key
    # (softmax weight 1) and all its rows give the same output, the tile's mean value; q-tile 1
    # keeps it.  Every row against the oracle.
    w = synth.Workload("sol-short", 100, 2, 17, 64, 0)
    bits = synth.qkv_bf16(w)
    bits["k"], bits["v"] = bits["k"][:40], bits["v"][:40]
    g = {t: gpu_u16(bits[t]) for t in bits}
    mask = np.ones((2, 2, 1), dtype=np.uint8)
    mask[:, 0, 0] = 0
    store = build_store(g["k"], g["v"]) if mode == "kvi8r" else None
    out = _run(mode, g["q"], g["k"], g["v"], store, 64, torch.from_numpy(mask).cuda())
    rows = np.arange(100)
    got, ref = [], []
    for h in range(2):
        got.append(_rows_out(out, rows, h))
        ref.append(_sol_ref(mode, lambda t, hh: bits[t][:, hh], store, h, rows, mask[h]))
    _assert_close(mode, np.concatenate(got), np.concatenate(ref), "sol-short")
    for h in range(2):
        first = got[h][:64]
        assert np.array_equal(first, np.broadcast_to(first[0], first.shape))
