"""Helpers shared by the GPU parity tests: host<->device copies of bit patterns,
store building through the C ABI, error metrics and oracle comparisons."""
from __future__ import annotations

import math

import numpy as np
import torch

import oracle
import store_kvi8r_quantize_amd as h3a
import synth

from parity import (CODE_MISMATCH, EXACT_REL_L2, KVI8R_MAX_ABS, KVI8R_REL_L2, SCALE,  # noqa: F401 (re-exported)
                    assert_quantize_ok, quantize_report, rel_l2)


def say(*a):
    print(*a, flush=True)


def gpu_u16(a: np.ndarray, dtype=torch.bfloat16) -> torch.Tensor:
    """uint16 bit patterns -> GPU tensor of a 16-bit dtype with the same bits."""
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to("cuda").view(dtype)


def host_u16(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def out_like(q: torch.Tensor, mode: str) -> torch.Tensor:
    """Output of an attention call: fp16 for the kvi8r stores (the precision kvi8r attention runs in, and the
    output the tolerances are stated for), bf16 for the exact store."""
    return torch.empty(q.shape, dtype=torch.float16 if mode in ("kvi8r", "kvi8r32") else torch.bfloat16,
                       device=q.device)


def out_f64(t: torch.Tensor) -> np.ndarray:
    """Exact fp64 values of an fp16 or bf16 output tensor."""
    bits = host_u16(t)
    return oracle.f16_to_f64(bits) if t.dtype == torch.float16 else oracle.bf16_to_f64(bits)


def gpu_inputs(w: synth.Workload, tensors=("q", "k", "v")) -> dict:
    """Token-major bf16 GPU tensors [S, H, 128], drawn head by head straight to the device."""
    import threading

    out = {t: torch.empty((w.seq, w.heads, 128), dtype=torch.bfloat16, device="cuda") for t in tensors}
    lock = threading.Lock()

    def sink(t, h, bits):
        src = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16)
        with lock:
            out[t][:, h, :].copy_(src)
            torch.cuda.synchronize()

    synth.for_each_head(w, tensors, sink)
    return out


class HeadSource:
    """Host bf16 bits of one (tensor, head), from token-major arrays or regenerated
    on demand (the tensors of the most recent head are kept)."""

    def __init__(self, w: synth.Workload, bits: dict | None = None):
        self.w, self.bits = w, bits
        self._head, self._val = None, {}

    def __call__(self, t: str, h: int) -> np.ndarray:
        if self.bits is not None:
            return self.bits[t][:, h]
        if self._head != h:
            self._head, self._val = h, {}
        if t not in self._val:
            self._val[t] = synth.head_bf16(self.w, t, h)
        return self._val[t]


def build_store(k: torch.Tensor, v: torch.Tensor, kv_chunk: int | None = None):
    """kvi8r store of token-major bf16 K/V [S, H, 128], built chunk by chunk."""
    s, nh, _ = k.shape
    kc, vc, sc = h3a.new_kvi8r_store(s, nh)
    step = kv_chunk or max(s, 1)
    for t0 in range(0, s, step):
        t1 = min(t0 + step, s)
        h3a.h3a_kv_quantize(k[t0:t1], kc, sc[0], token_offset=t0)
        h3a.h3a_kv_quantize(v[t0:t1], vc, sc[1], token_offset=t0)
    return kc, vc, sc


def store_head(kc, vc, sc, h):
    """Host copies of one head of a kvi8r store: (k codes, k scale bits, v codes, v scale bits)."""
    return (kc[h].cpu().numpy(), host_u16(sc[0, h]), vc[h].cpu().numpy(), host_u16(sc[1, h]))


def oracle_exact_rows(src: HeadSource, h, rows, mask=None):
    k = src("k", h)
    keep = None if mask is None else oracle.expand_tile_mask(mask[h], rows, k.shape[0])
    q = src("q", h)[rows]
    return oracle.exact_attention_bf16(q, k, src("v", h), SCALE, keep)


def oracle_kvi8r_rows(src: HeadSource, store_h, h, rows, mask=None):
    kc, ks, vc, vs = store_h
    keep = None if mask is None else oracle.expand_tile_mask(mask[h], rows, kc.shape[0])
    return oracle.kvi8r_attention(oracle.bf16_to_f64(src("q", h)[rows]), kc, ks, vc, vs, SCALE, keep)


def out_rows(out_gpu_bits: np.ndarray, h, rows) -> np.ndarray:
    return oracle.bf16_to_f64(out_gpu_bits[rows, h])


def pool_check(pool, kind, w, out, heads, rows_of, store=None, mask=None, tag="", s_kv=None):
    """Compare GPU output rows with the fp64 oracle, one head per pool job, gates per head and pooled.

    kind: "exact", "kvi8r", "sol_exact" or "sol_kvi8r"; store: the GPU's kvi8r store (k codes, v codes,
    scales) for kvi8r kinds; mask: the tile mask [H, nQt, nKt] for masked kinds.
    """
    from parity import assert_attention_ok, attention_job

    specs = []
    for h in heads:
        rows = np.asarray(rows_of(h))
        spec = {"kind": kind, "workload": w, "head": h, "rows": rows, "s_kv": s_kv,
                "got": host_u16(out[torch.from_numpy(rows).cuda(), h]), "got_f16": out.dtype == torch.float16}
        if store is not None:
            spec["store"] = store_head(*store, h)
        if mask is not None:
            spec["mask"] = np.ascontiguousarray(mask[h])
        specs.append(spec)
    results = []
    for r in pool.ex.map(attention_job, specs):
        say(tag, kind, "head", r["head"], "rows", r["rows"], "relL2", r["rel_l2"], "max abs", r["max_abs"])
        results.append(r)
    gate = {"sol_exact": "exact", "sol_kvi8r": "kvi8r"}.get(kind, kind)
    if gate == "kvi8r" and out.dtype == torch.bfloat16:
        gate = "kvi8r_bf16"
    summary = assert_attention_ok(results, gate)
    say(tag, kind, "summary", summary)
    return summary
