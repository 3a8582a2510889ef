"""GPU parity of chunked attention (through the C ABI) against the fp64 oracle.

kvi8r: relative L2 <= 2e-3 and max abs <= 1e-2 against the oracle on the GPU's
own store (identically dequantised K/V).  Exact: relative L2 <= 4e-3 against
the unquantised inputs, and bitwise identical across q_chunk and kv_block
("H3 Streamed Blocks" node page, Inputs table: q_chunk "exact at any value";
kv_block).  Tile mask: an all-ones mask reproduces dense attention bitwise,
dropped tiles are excluded, a row with nothing kept is zero ("H3-Optimizations"
page, Nodes).
"""
import numpy as np
import pytest
import torch

import oracle
import store_kvi8r_quantize_amd as h3a
import synth
from gpu_common import (EXACT_REL_L2, KVI8R_MAX_ABS, KVI8R_REL_L2, HeadSource, build_store, gpu_inputs, gpu_u16,
                        host_u16, oracle_exact_rows, oracle_kvi8r_rows, out_f64, out_like, pool_check, rel_l2, say,
                        store_head)

pytestmark = pytest.mark.gpu

_CACHE = {}


def _inputs(name):
    """(workload, host head source, GPU tensors); one workload cached at a time."""
    if name not in _CACHE:
        w = synth.WORKLOADS[name]
        say("generating", name)
        _CACHE.clear()
        torch.cuda.empty_cache()
        if w.seq * w.heads <= 16384 * 8:
            bits = synth.qkv_bf16(w)
            _CACHE[name] = (w, HeadSource(w, bits), {t: gpu_u16(bits[t]) for t in bits})
        else:
            _CACHE[name] = (w, HeadSource(w), gpu_inputs(w))
    return _CACHE[name]


def _run(mode, q, k, v, store=None, q_chunk=256, kv_block=0, mask=None, out_dtype=None):
    out = out_like(q, mode) if out_dtype is None else torch.empty(q.shape, dtype=out_dtype, device=q.device)
    if mode == "kvi8r":
        kc, vc, sc = store
        h3a.h3a_attention(q, kc, vc, sc, out, q_chunk=q_chunk, kv_block=kv_block, mode="kvi8r", tile_mask=mask)
    else:
        h3a.h3a_attention(q, k, v, None, out, q_chunk=q_chunk, kv_block=kv_block, mode="exact", tile_mask=mask)
    torch.cuda.synchronize()
    return out


def _check(mode, heads, src, out, store, rows_of, mask=None, tag=""):
    worst, mx = 0.0, 0.0
    got_all, ref_all = [], []
    heads = range(heads) if isinstance(heads, int) else heads
    for h in heads:
        rows = rows_of(h)
        if mode == "kvi8r":
            ref = oracle_kvi8r_rows(src, store_head(*store, h), h, rows, mask)
        else:
            ref = oracle_exact_rows(src, h, rows, mask)
        got = out_f64(out[torch.from_numpy(rows).cuda(), h])
        r = rel_l2(got, ref)
        worst = max(worst, r)
        mx = max(mx, float(np.abs(got - ref).max()))
        got_all.append(got)
        ref_all.append(ref)
    total = rel_l2(np.concatenate(got_all), np.concatenate(ref_all))
    say(tag, mode, "relL2", total, "worst head", worst, "max abs", mx)
    # the gates hold on every head (worst) and over all rows together
    if mode == "kvi8r":
        assert total <= KVI8R_REL_L2 and worst <= KVI8R_REL_L2 and mx <= KVI8R_MAX_ABS
    else:
        assert total <= EXACT_REL_L2 and worst <= EXACT_REL_L2
    return total, worst, mx


@pytest.mark.parametrize("mode", ["exact", "kvi8r"])
def test_tiny_all_rows(mode):
    w, bits, g = _inputs("tiny")
    store = build_store(g["k"], g["v"], kv_chunk=w.q_chunk) if mode == "kvi8r" else None
    out = _run(mode, g["q"], g["k"], g["v"], store, q_chunk=w.q_chunk, kv_block=w.kv_block)
    _check(mode, w.heads, bits, out, store, lambda h: np.arange(w.seq), tag="tiny")


@pytest.mark.timeout(600)
@pytest.mark.parametrize("mode", ["exact", "kvi8r"])
def test_outlier16k_all_rows(mode, oracle_pool):
    # every row of every head (16384 x 8) against the fp64 oracle
    w, bits, g = _inputs("outlier16k")
    store = build_store(g["k"], g["v"], kv_chunk=w.q_chunk) if mode == "kvi8r" else None
    out = _run(mode, g["q"], g["k"], g["v"], store, q_chunk=w.q_chunk, kv_block=w.kv_block)
    pool_check(oracle_pool, mode, w, out, range(w.heads), lambda h: np.arange(w.seq), store, tag="outlier16k")


@pytest.mark.parametrize("mode", ["exact", "kvi8r"])
@pytest.mark.parametrize("s_q,s_kv,heads,q_chunk", [(1000, 777, 3, 300), (65, 1, 2, 64), (257, 129, 1, 1000),
                                                     (130, 200, 96, 64)])  # wide token stride, ragged last tile
def test_ragged_shapes(mode, s_q, s_kv, heads, q_chunk):
    w = synth.Workload("ragged", max(s_q, s_kv), heads, 7, q_chunk, 0)
    full = synth.qkv_bf16(w)
    bits = {"q": full["q"][:s_q], "k": full["k"][:s_kv], "v": full["v"][:s_kv]}
    g = {t: gpu_u16(bits[t]) for t in bits}
    store = build_store(g["k"], g["v"]) if mode == "kvi8r" else None
    out = _run(mode, g["q"], g["k"], g["v"], store, q_chunk=q_chunk)
    _check(mode, heads, HeadSource(w, bits), out, store, lambda h: np.arange(s_q), tag=f"ragged{s_q}x{s_kv}")


def test_single_key_returns_value_row_exactly():
    w = synth.Workload("one", 300, 2, 8, 128, 0)
    bits = synth.qkv_bf16(w)
    q, k, v = gpu_u16(bits["q"]), gpu_u16(bits["k"][:1]), gpu_u16(bits["v"][:1])
    out = _run("exact", q, k, v, q_chunk=128)
    assert np.array_equal(host_u16(out), np.broadcast_to(bits["v"][:1], bits["q"].shape))


@pytest.mark.parametrize("mode", ["exact", "kvi8r"])
def test_no_keys_gives_zero(mode):
    q = gpu_u16(synth.qkv_bf16(synth.Workload("z", 100, 2, 9, 64, 0), ("q",))["q"])
    if mode == "kvi8r":
        store = h3a.new_kvi8r_store(0, 2)
        out = torch.ones_like(q)
        h3a.h3a_attention(q, store[0], store[1], store[2], out, q_chunk=64, mode="kvi8r")
    else:
        e = torch.empty((0, 2, 128), dtype=torch.bfloat16, device="cuda")
        out = torch.ones_like(q)
        h3a.h3a_attention(q, e, e, None, out, q_chunk=64, mode="exact")
    torch.cuda.synchronize()
    assert not bool(out.any())


@pytest.mark.parametrize("mode", ["exact", "kvi8r"])
def test_zero_query_averages_values(mode):
    w, src, g = _inputs("tiny")
    q = torch.zeros_like(g["q"])
    store = build_store(g["k"], g["v"]) if mode == "kvi8r" else None
    out = _run(mode, q, g["k"], g["v"], store)
    got = out_f64(out)
    for h in range(w.heads):
        if mode == "kvi8r":
            kc, ks, vc, vs = store_head(*store, h)
            want = oracle.dequantize_rows(vc, vs).mean(axis=0) @ oracle.orthonormal_hadamard()
        else:
            want = oracle.bf16_to_f64(src("v", h)).mean(axis=0)
        assert rel_l2(got[:, h], np.broadcast_to(want, got[:, h].shape)) < 4e-3


@pytest.mark.parametrize("mode", ["exact", "kvi8r"])
def test_q_chunk_and_kv_block_bitwise_invariance(mode):
    w, bits, g = _inputs("outlier64k")
    store = build_store(g["k"], g["v"], kv_chunk=w.q_chunk) if mode == "kvi8r" else None
    base = _run(mode, g["q"], g["k"], g["v"], store, q_chunk=16384, kv_block=16384)
    for q_chunk, kv_block in ((1024, 16384), (4096, 16384), (16384, 0), (4096, 4096), (1000, 64)):
        other = _run(mode, g["q"], g["k"], g["v"], store, q_chunk=q_chunk, kv_block=kv_block)
        same = torch.equal(base.view(torch.int16), other.view(torch.int16))
        say("outlier64k", mode, "q_chunk", q_chunk, "kv_block", kv_block, "bitwise equal", same)
        assert same



@pytest.mark.timeout(600)
def test_kvi8r_bf16_output(oracle_pool):
    # The kvi8r store's output delivered in bf16 (the model dtype) is the same fp32 value rounded to bf16
    # instead of fp16: elementwise the two differ by at most half an ulp of each format, and against the
    # oracle the bf16 output keeps relative L2 <= 2e-3 (every row of outlier16k).
    w, bits, g = _inputs("outlier16k")
    store = build_store(g["k"], g["v"], kv_chunk=w.q_chunk)
    f16 = _run("kvi8r", g["q"], g["k"], g["v"], store, q_chunk=w.q_chunk)
    b16 = _run("kvi8r", g["q"], g["k"], g["v"], store, q_chunk=w.q_chunk, out_dtype=torch.bfloat16)
    f, b = out_f64(f16), out_f64(b16)
    from parity import half_ulp

    top = np.maximum(np.abs(f), np.abs(b))
    excess = np.abs(b - f) - half_ulp(top, 7) - half_ulp(top, 10)
    say("kvi8r bf16 vs fp16 output: max |b - f|", float(np.abs(b - f).max()), "max excess", float(excess.max()))
    assert np.all(excess <= 0)
    pool_check(oracle_pool, "kvi8r", w, b16, range(w.heads), lambda h: np.arange(w.seq), store,
               tag="outlier16k-bf16-out")


@pytest.mark.timeout(900)
@pytest.mark.parametrize("mode", ["exact", "kvi8r"])
def test_outlier64k_oracle_sample(mode, oracle_pool):
    # the configuration's 2048 seeded rows on every one of the 32 heads
    w, bits, g = _inputs("outlier64k")
    store = build_store(g["k"], g["v"], kv_chunk=w.q_chunk) if mode == "kvi8r" else None
    out = _run(mode, g["q"], g["k"], g["v"], store, q_chunk=w.q_chunk, kv_block=w.kv_block)
    pool_check(oracle_pool, mode, w, out, range(w.heads), lambda h: synth.sampled_rows(w, h), store,
               tag="outlier64k")


@pytest.mark.parametrize("mode", ["exact", "kvi8r"])
def test_all_ones_mask_equals_dense_bitwise(mode):
    w, bits, g = _inputs("outlier16k")
    store = build_store(g["k"], g["v"]) if mode == "kvi8r" else None
    nt = w.n_tiles
    ones = torch.ones((w.heads, nt, nt), dtype=torch.uint8, device="cuda")
    dense = _run(mode, g["q"], g["k"], g["v"], store, q_chunk=4096)
    sparse = _run(mode, g["q"], g["k"], g["v"], store, q_chunk=4096, mask=ones)
    assert torch.equal(dense.view(torch.int16), sparse.view(torch.int16))


@pytest.mark.parametrize("mode", ["exact", "kvi8r"])
def test_random_mask_with_empty_tiles(mode):
    w = synth.Workload("masked", 1000, 2, 12, 256, 0)
    bits = synth.qkv_bf16(w)
    g = {t: gpu_u16(bits[t]) for t in bits}
    nt = w.n_tiles
    rng = np.random.default_rng(4)
    mask = (rng.random((2, nt, nt)) < 0.3).astype(np.uint8)
    mask[:, 3, :] = 0  # rows 192..255 keep nothing
    store = build_store(g["k"], g["v"]) if mode == "kvi8r" else None
    out = _run(mode, g["q"], g["k"], g["v"], store, q_chunk=256, mask=torch.from_numpy(mask).cuda())
    assert not bool(out[192:256].any())
    _check(mode, w.heads, HeadSource(w, bits), out, store, lambda h: np.arange(w.seq), mask=mask, tag="masked")


@pytest.mark.timeout(900)
@pytest.mark.parametrize("mode", ["kvi8r", "exact"])
def test_sparse64k_oracle_sample(mode, oracle_pool):
    # every text q-tile (8) plus 24 seeded video q-tiles of each of the 32 heads: 2048 rows per head
    w, bits, g = _inputs("sparse64k")
    mask = synth.tile_mask(w)
    store = build_store(g["k"], g["v"], kv_chunk=w.q_chunk) if mode == "kvi8r" else None
    out = _run(mode, g["q"], g["k"], g["v"], store, q_chunk=w.q_chunk, mask=torch.from_numpy(mask).cuda())
    pool_check(oracle_pool, mode, w, out, range(w.heads), lambda h: synth.q_tile_rows(w, synth.sampled_q_tiles(w, h)),
               store, mask=mask, tag="sparse64k")


@pytest.mark.timeout(1200)
@pytest.mark.parametrize("mode", ["kvi8r", "exact"])
def test_long217k_oracle_sample(mode, oracle_pool):
    # the configuration's 2048 seeded rows on every one of the 32 heads, against all 217088 keys
    w, bits, g = _inputs("long217k")
    store = build_store(g["k"], g["v"], kv_chunk=w.q_chunk) if mode == "kvi8r" else None
    out = _run(mode, g["q"], g["k"], g["v"], store, q_chunk=w.q_chunk, kv_block=w.kv_block)
    pool_check(oracle_pool, mode, w, out, range(w.heads), lambda h: synth.sampled_rows(w, h), store, tag="long217k")


@pytest.mark.parametrize("raw_handle", [False, True])
def test_side_stream_with_binding_workspace(raw_handle):
    # The binding allocates the workspace (workspace=None) for kernels queued on a side stream, then the
    # current stream immediately allocates and fills memory of the same size.  The workspace belongs to the
    # side stream's pool, so that churn cannot take its block while the kernels run: the output is bitwise
    # that of the same call on the current stream.
    w, bits, g = _inputs("outlier16k")
    store = build_store(g["k"], g["v"])
    ref = _run("kvi8r", g["q"], g["k"], g["v"], store, q_chunk=4096)
    need = h3a.h3a_attention_workspace_bytes(w.seq, w.seq, w.heads, 4096, "kvi8r", False)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    out = out_like(g["q"], "kvi8r")
    for _ in range(3):
        h3a.h3a_attention(g["q"], *store, out, q_chunk=4096, mode="kvi8r",
                          stream=side.cuda_stream if raw_handle else side)
        junk = [torch.full((need,), 0x7F, dtype=torch.uint8, device="cuda") for _ in range(2)]
        del junk
    side.synchronize()
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))


@pytest.mark.parametrize("mode", ["exact", "kvi8r"])
@pytest.mark.parametrize("q_chunk", [192, 64, 320])
def test_mask_chunks_of_odd_q_tile_counts(mode, q_chunk):
    # Chunks of 3, 1 and 5 routing q-tiles; q-tile 4 keeps nothing while q-tile 5 keeps about half its
    # tiles; q-tiles 6 and 7 keep the same tiles; the ragged last KV tile (s_kv = 1000) is kept by every
    # other q-tile.  All rows against the oracle, and bitwise equal to q_chunk 128 (each row's tile sequence
    # does not depend on how rows are grouped into chunks).
    w = synth.Workload("odd-chunks", 1000, 3, 14, q_chunk, 0)
    bits = synth.qkv_bf16(w)
    g = {t: gpu_u16(bits[t]) for t in bits}
    nt = w.n_tiles
    rng = np.random.default_rng(21)
    mask = (rng.random((3, nt, nt)) < 0.3).astype(np.uint8)
    mask[:, 4, :] = 0
    mask[:, 5, :] = (rng.random((3, nt)) < 0.5)
    mask[:, 6, :] = mask[:, 7, :]
    mask[:, :, nt - 1] = 1  # the partial tile is kept everywhere but q-tile 4
    mask[:, 4, :] = 0
    store = build_store(g["k"], g["v"]) if mode == "kvi8r" else None
    m = torch.from_numpy(mask).cuda()
    out = _run(mode, g["q"], g["k"], g["v"], store, q_chunk=q_chunk, mask=m)
    ref = _run(mode, g["q"], g["k"], g["v"], store, q_chunk=128, mask=m)
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
    assert not bool(out[256:320].any())
    _check(mode, w.heads, HeadSource(w, bits), out, store, lambda h: np.arange(w.seq), mask=mask, tag="odd-chunks")


@pytest.mark.parametrize("mode", ["exact", "kvi8r"])
def test_mask_lists_of_one_tile_and_the_partial_tile_alone(mode):
    # 1000 keys: 15 whole tiles and a partial 16th (40 keys).  q-tile 0 keeps only the partial tile (no whole
    # tile before it), q-tile 1 only tile 0, q-tile 2 tile 0 and the partial one, q-tile 3 nothing, q-tile 4
    # every tile; the exact store's paired kernel then runs pairs of unequal list lengths with the partial tile
    # in one list of the pair only.  All rows against the oracle.
    w = synth.Workload("short-lists", 1000, 2, 15, 256, 0)
    bits = synth.qkv_bf16(w)
    g = {t: gpu_u16(bits[t]) for t in bits}
    nt = w.n_tiles
    mask = np.zeros((2, nt, nt), dtype=np.uint8)
    mask[:, 0, nt - 1] = 1
    mask[:, 1, 0] = 1
    mask[:, 2, [0, nt - 1]] = 1
    mask[:, 4, :] = 1
    rng = np.random.default_rng(5)
    mask[:, 5:, :] = (rng.random((2, nt - 5, nt)) < 0.3)
    store = build_store(g["k"], g["v"]) if mode == "kvi8r" else None
    out = _run(mode, g["q"], g["k"], g["v"], store, q_chunk=256, mask=torch.from_numpy(mask).cuda())
    assert not bool(out[192:256].any())
    _check(mode, w.heads, HeadSource(w, bits), out, store, lambda h: np.arange(w.seq), mask=mask, tag="short-lists")
