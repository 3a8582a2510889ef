"""GPU parity of per-row store routing (h3a_attention_routed, through the C ABI).

"H3 Streamed Blocks" node page, Inputs table, exact_av_rows row: text and audio
query rows attend a retained bf16 K/V exactly, the other rows the quantised
store.  Every row's result depends only on that row and its store, so a routed
row must equal, bit for bit, the row that h3a_attention gives it in its mode;
the small cases are also compared with the oracle (oracle/routing.py) at the
tolerances of each mode.
"""
import numpy as np
import pytest
import torch

import oracle
import store_kvi8r_quantize_amd as h3a
import synth
from gpu_common import (EXACT_REL_L2, KVI8R_MAX_ABS, KVI8R_REL_L2, SCALE, build_store, gpu_inputs, gpu_u16, host_u16,
                        rel_l2, say, store_head)

pytestmark = pytest.mark.gpu


def _full(mode, q, k, v, store, q_chunk):
    out = torch.empty_like(q)
    if mode == "kvi8r":
        h3a.h3a_attention(q, *store, out, q_chunk=q_chunk, mode="kvi8r")
    else:
        h3a.h3a_attention(q, k, v, None, out, q_chunk=q_chunk, mode="exact")
    return out


def _routed(q, k, v, store, spans, q_chunk):
    out = torch.empty_like(q)
    h3a.h3a_attention_routed(q, k, v, store, out, exact_spans=spans, q_chunk=q_chunk)
    torch.cuda.synchronize()
    return out


def _assert_rows_follow_modes(out, exact, quant, spans):
    rows = torch.from_numpy(oracle.spans_to_rows(spans, out.shape[0])).cuda()
    o, e, r = (t.view(torch.int16) for t in (out, exact, quant))
    assert torch.equal(o[rows], e[rows])
    assert torch.equal(o[~rows], r[~rows])


@pytest.mark.parametrize("s,s_kv,heads,q_chunk,spans", [
    (1024, 1024, 2, 256, [(0, 100), (300, 301), (700, 1024)]),
    (1000, 777, 3, 300, [(5, 5), (64, 640)]),
    (257, 129, 1, 1000, [(256, 257)]),
    (1000, 777, 3, 256, []),
    (1000, 777, 3, 256, [(0, 1000)]),
])
def test_routed_rows_equal_their_mode_bitwise(s, s_kv, heads, q_chunk, spans):
    w = synth.Workload("routed", max(s, s_kv), heads, 31, 256, 0)
    bits = synth.qkv_bf16(w)
    q = gpu_u16(bits["q"][:s])
    k, v = gpu_u16(bits["k"][:s_kv]), gpu_u16(bits["v"][:s_kv])
    store = build_store(k, v)
    out = _routed(q, k, v, store, spans, q_chunk)
    _assert_rows_follow_modes(out, _full("exact", q, k, v, None, q_chunk), _full("kvi8r", q, k, v, store, q_chunk),
                              spans)


def test_routed_against_oracle():
    w = synth.WORKLOADS["tiny"]
    bits = synth.qkv_bf16(w)
    g = {t: gpu_u16(bits[t]) for t in bits}
    store = build_store(g["k"], g["v"], kv_chunk=w.q_chunk)
    spans = [(0, 90), (500, 777)]
    out = _routed(g["q"], g["k"], g["v"], store, spans, w.q_chunk)
    rows = oracle.spans_to_rows(spans, w.seq)
    got_all, ref_all = [], []
    for h in range(w.heads):
        kc, ks, vc, vs = store_head(*store, h)
        ref = oracle.routed_attention(bits["q"][:, h], bits["k"][:, h], bits["v"][:, h], kc, ks, vc, vs, SCALE, rows)
        got_all.append(oracle.bf16_to_f64(host_u16(out[:, h])))
        ref_all.append(ref)
    got, ref = np.stack(got_all, 1), np.stack(ref_all, 1)
    re = rel_l2(got[rows], ref[rows])
    rq = rel_l2(got[~rows], ref[~rows])
    # routed output is bf16 for every row: kvi8r rows get the two half-ulps that separate it from fp16
    from parity import half_ulp

    dq = np.abs(got[~rows] - ref[~rows]) - half_ulp(ref[~rows], 7) - half_ulp(ref[~rows], 10)
    mq = float(dq.max())
    say("routed tiny: exact rows relL2", re, "kvi8r rows relL2", rq, "max abs beyond the bf16 rounding", mq)
    assert re <= EXACT_REL_L2
    assert rq <= KVI8R_REL_L2 and mq <= KVI8R_MAX_ABS


@pytest.mark.timeout(600)
def test_routed_long217k_text_and_audio_spans():
    # 217088 rows: a 5760-row text prefix and a 2240-row audio tail attend exactly (3.7 % of rows,
    # the share the node page gives for text + audio), the video rows in between attend the kvi8r store.
    w = synth.WORKLOADS["long217k"]
    say("generating", w.name)
    g = gpu_inputs(w)
    store = build_store(g["k"], g["v"], kv_chunk=w.q_chunk)
    spans = [(0, 5760), (w.seq - 2240, w.seq)]
    out = _routed(g["q"], g["k"], g["v"], store, spans, w.q_chunk)
    exact = _full("exact", g["q"], g["k"], g["v"], None, w.q_chunk)
    quant = _full("kvi8r", g["q"], g["k"], g["v"], store, w.q_chunk)
    torch.cuda.synchronize()
    _assert_rows_follow_modes(out, exact, quant, spans)
