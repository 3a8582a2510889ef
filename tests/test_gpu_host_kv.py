"""GPU parity of host-staged K/V (h3a_attention_host_kv, through the C ABI).

"H3 Streamed Blocks" node page, Inputs table, kv_block row: K/V attended in
blocks with a log-sum-exp combine, kept for a host-staged K/V store.  The store
sits in pinned host memory and reaches the GPU one kv_block at a time; each
block's launch carries every row's running (m, l, O) through the workspace.
Carrying that state is exact and the tile order is the same, so the output must
equal, bit for bit, h3a_attention over the same store resident on the GPU (which
the attention tests compare with the oracle); the tiny case is also compared
with the oracle directly.
"""
import numpy as np
import pytest
import torch

import oracle
import store_kvi8r_quantize_amd as h3a
import synth
from gpu_common import (KVI8R_MAX_ABS, KVI8R_REL_L2, SCALE, build_store, gpu_inputs, gpu_u16, host_u16, out_f64,
                        out_like, rel_l2, say, store_head)

pytestmark = pytest.mark.gpu


def _pinned(t):
    h = torch.empty(t.shape, dtype=t.dtype, pin_memory=True)
    h.copy_(t)
    return h


def _store(mode, k, v, kv_chunk=None):
    if mode == "exact":
        return k, v, None
    kc, vc, sc = h3a.new_kvi8r_store(k.shape[0], k.shape[1], per32=(mode == "kvi8r32"))
    step = kv_chunk or max(k.shape[0], 1)
    for t0 in range(0, k.shape[0], step):
        h3a.h3a_kv_quantize(k[t0:t0 + step], kc, sc[0], token_offset=t0)
        h3a.h3a_kv_quantize(v[t0:t0 + step], vc, sc[1], token_offset=t0)
    return kc, vc, sc


def _device(mode, q, store, q_chunk):
    out = out_like(q, mode)
    h3a.h3a_attention(q, *store, out, q_chunk=q_chunk, mode=mode)
    return out


def _staged(mode, q, store, q_chunk, kv_block):
    host = [None if t is None else _pinned(t) for t in store]
    torch.cuda.synchronize()
    out = out_like(q, mode)
    h3a.h3a_attention_host_kv(q, *host, out, q_chunk=q_chunk, kv_block=kv_block, mode=mode)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("mode", ["exact", "kvi8r", "kvi8r32"])
@pytest.mark.parametrize("s,s_kv,heads,q_chunk,kv_block", [
    (1024, 1024, 2, 256, 256),    # 4 full blocks
    (1000, 777, 3, 300, 128),     # 7 blocks, the last one of 9 keys; ragged query chunks
    (257, 129, 1, 1000, 4096),    # one block holding the whole store
    (65, 1, 2, 64, 64),           # a single key
    (300, 640, 2, 128, 0),        # kv_block 0: the default 16384, one block
    (300, 0, 2, 128, 64),         # an empty store: every row is zero, as on the device
])
def test_staged_equals_device_resident_bitwise(mode, s, s_kv, heads, q_chunk, kv_block):
    w = synth.Workload("staged", max(s, s_kv), heads, 51, 256, 0)
    bits = synth.qkv_bf16(w)
    q = gpu_u16(bits["q"][:s])
    store = _store(mode, gpu_u16(bits["k"][:s_kv]), gpu_u16(bits["v"][:s_kv]))
    dev = _device(mode, q, store, q_chunk)
    got = _staged(mode, q, store, q_chunk, kv_block)
    assert torch.equal(got.view(torch.int16), dev.view(torch.int16))


def test_staged_kvi8r_against_oracle():
    w = synth.WORKLOADS["tiny"]
    bits = synth.qkv_bf16(w)
    g = {t: gpu_u16(bits[t]) for t in bits}
    store = build_store(g["k"], g["v"], kv_chunk=w.q_chunk)
    out = _staged("kvi8r", g["q"], store, w.q_chunk, 192)
    got_all, ref_all = [], []
    for h in range(w.heads):
        kc, ks, vc, vs = store_head(*store, h)
        ref_all.append(oracle.kvi8r_attention(oracle.bf16_to_f64(bits["q"][:, h]), kc, ks, vc, vs, SCALE))
        got_all.append(out_f64(out[:, h]))
    got, ref = np.concatenate(got_all), np.concatenate(ref_all)
    r, mx = rel_l2(got, ref), float(np.abs(got - ref).max())
    say("staged tiny kvi8r relL2", r, "max abs", mx)
    assert r <= KVI8R_REL_L2 and mx <= KVI8R_MAX_ABS


def test_staged_rejects_pageable_and_short_host_buffers():
    w = synth.Workload("staged-bad", 256, 2, 52, 256, 0)
    bits = synth.qkv_bf16(w)
    q = gpu_u16(bits["q"])
    k, v = gpu_u16(bits["k"]), gpu_u16(bits["v"])
    out = torch.empty_like(q)
    lib = h3a.library()
    ws = torch.empty(max(h3a.h3a_attention_host_kv_workspace_bytes(256, 256, 2, 256, 64, "exact"), 256),
                     dtype=torch.uint8, device="cuda")
    pageable = k.cpu()
    rc = lib.h3a_attention_host_kv(q.data_ptr(), pageable.data_ptr(), pageable.data_ptr(), None, 256, 256, 2, 128,
                                   SCALE, 256, 64, 0, out.data_ptr(), ws.data_ptr(), ws.numel(), None)
    assert rc == -1 and "pinned" in lib.h3a_last_error().decode()
    short = _pinned(k[:50])  # 50 tokens where 256 are needed (the pinned allocator rounds sizes up)
    rc = lib.h3a_attention_host_kv(q.data_ptr(), short.data_ptr(), short.data_ptr(), None, 256, 256, 2, 128,
                                   SCALE, 256, 64, 0, out.data_ptr(), ws.data_ptr(), ws.numel(), None)
    err = lib.h3a_last_error().decode()
    say("short pinned buffer:", rc, err)
    assert rc == -1 and "k_host" in err
    # the well-formed call still works after the rejected ones
    got = _staged("exact", q, (k, v, None), 256, 64)
    assert torch.equal(got.view(torch.int16), _device("exact", q, (k, v, None), 256).view(torch.int16))


@pytest.mark.timeout(600)
def test_staged_long217k_kvi8r_bitwise():
    w = synth.WORKLOADS["long217k"]
    say("generating", w.name)
    g = gpu_inputs(w)
    store = build_store(g["k"], g["v"], kv_chunk=w.q_chunk)
    del g["k"], g["v"]
    dev = _device("kvi8r", g["q"], store, w.q_chunk)
    got = _staged("kvi8r", g["q"], store, w.q_chunk, w.kv_block)
    assert torch.equal(got.view(torch.int16), dev.view(torch.int16))


@pytest.mark.timeout(600)
@pytest.mark.parametrize("mode", ["exact", "kvi8r"])
def test_staged_long217k_wide_q_chunk_bitwise(mode):
    """The bench's wider host-staged setting: q_chunk 65536 (four query chunks, so four passes of the store
    over PCIe) gives the bits of the resident call at q_chunk 16384."""
    w = synth.WORKLOADS["long217k"]
    say("generating", w.name, "mode", mode)
    g = gpu_inputs(w)
    if mode == "kvi8r":
        store = build_store(g["k"], g["v"], kv_chunk=w.q_chunk)
        del g["k"], g["v"]
    else:
        store = (g.pop("k"), g.pop("v"), None)
    dev = _device(mode, g["q"], store, w.q_chunk)
    got = _staged(mode, g["q"], store, 65536, w.kv_block)
    assert torch.equal(got.view(torch.int16), dev.view(torch.int16))
