"""h3a_attention_noalloc (no workspace: the library's own per-GPU scratch) against
h3a_attention with a caller workspace, through the C ABI.

Both run the same kernels at the same q_chunk, so the outputs must be bitwise
equal (stricter than the oracle tolerances of the attention tests).  Two calls
in a row, the second on a smaller input, so the second runs over scratch the
first left behind; then a request above the scratch size is refused.
"""
import numpy as np
import pytest
import torch

import store_kvi8r_quantize_amd as h3a
import synth
from gpu_common import gpu_u16, say

pytestmark = pytest.mark.gpu


def _case(seq, heads, seed, mode, q_chunk, masked):
    w = synth.Workload(f"noalloc{seq}", seq, heads, seed, q_chunk, 0, k_outliers=True)
    bits = synth.qkv_bf16(w)
    g = {t: gpu_u16(bits[t]) for t in bits}
    if mode == "exact":
        store = (g["k"], g["v"], None)
    else:
        kc, vc, sc = h3a.new_kvi8r_store(seq, heads, per32=mode == "kvi8r32")
        h3a.h3a_kv_quantize(g["k"], kc, sc[0])
        h3a.h3a_kv_quantize(g["v"], vc, sc[1])
        store = (kc, vc, sc)
    mask = None
    if masked:
        rng = np.random.default_rng(seed)
        m = (rng.random((heads, w.n_tiles, w.n_tiles)) < 0.3).astype(np.uint8)
        m[:, 0, :] = 0  # one q-tile keeps nothing
        mask = torch.from_numpy(m).cuda()
    return g["q"], store, mask


def _both(q, store, mask, mode, q_chunk, sol):
    ref = torch.full_like(q, 3.0)
    got = torch.full_like(q, -5.0)
    h3a.h3a_attention(q, *store, ref, q_chunk=q_chunk, mode=mode, tile_mask=mask, sol=sol)
    h3a.h3a_attention_noalloc(q, *store, got, q_chunk=q_chunk, mode=mode, tile_mask=mask, sol=sol)
    torch.cuda.synchronize()
    return ref, got


@pytest.mark.parametrize("mode,masked,sol", [("kvi8r", False, False), ("kvi8r", True, True), ("exact", True, False),
                                             ("kvi8r32", False, False)])
def test_noalloc_equals_workspace_call_twice(mode, masked, sol):
    for seq, heads, q_chunk in ((4096, 8, 1024), (1000, 2, 256)):  # the second call is the smaller one
        q, store, mask = _case(seq, heads, 40 + heads, mode, q_chunk, masked)
        ref, got = _both(q, store, mask, mode, q_chunk, sol)
        same = torch.equal(ref.view(torch.int16), got.view(torch.int16))
        say("noalloc", mode, "masked" if masked else "dense", "sol" if sol else "", seq, heads, "bitwise equal", same)
        assert same


def test_noalloc_refuses_more_than_its_scratch():
    q = torch.zeros((16384, 32, 128), dtype=torch.bfloat16, device="cuda")
    kc, vc, sc = h3a.new_kvi8r_store(64, 32)
    out = torch.zeros_like(q)
    with pytest.raises(h3a.H3AError, match="h3a_attention_noalloc"):
        h3a.h3a_attention_noalloc(q, kc, vc, sc, out, q_chunk=16384, mode="kvi8r")
    torch.cuda.synchronize()
    assert not bool(out.any())  # nothing was queued
