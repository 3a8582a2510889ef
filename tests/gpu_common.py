"""Helpers shared by the GPU parity tests: host<->device copies of bit patterns,
store building through the C ABI, error metrics and oracle comparisons."""
from __future__ import annotations

import math

import numpy as np
import torch

import oracle
import store_kvi8r_quantize_amd as h3a
import synth

SCALE = 1.0 / math.sqrt(128.0)

# Tolerances stated for this path: kvi8r output against the oracle on the same
# dequantised K/V: relative L2 <= 2e-3 and max abs <= 1e-2; exact path against
# the unquantised inputs: relative L2 <= 4e-3.  Codes: <= 1e-4 off by one (ties);
# scales within 1 fp16 ulp.
KVI8R_REL_L2 = 2e-3
KVI8R_MAX_ABS = 1e-2
EXACT_REL_L2 = 4e-3
CODE_MISMATCH = 1e-4


def say(*a):
    print(*a, flush=True)


def gpu_u16(a: np.ndarray, dtype=torch.bfloat16) -> torch.Tensor:
    """uint16 bit patterns -> GPU tensor of a 16-bit dtype with the same bits."""
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to("cuda").view(dtype)


def host_u16(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def rel_l2(got, ref) -> float:
    d = np.linalg.norm(np.asarray(got, np.float64) - ref)
    n = np.linalg.norm(ref)
    return float(d / n) if n > 0 else float(d)


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


def quantize_report(x_bits: np.ndarray, codes_gpu: np.ndarray, scale_bits_gpu: np.ndarray, group: int = 128) -> dict:
    """Compare one head's GPU codes and scales with the oracle.

    x_bits: bf16 bits [n, 128]; codes_gpu: int8 [n, 128]; scale_bits_gpu: [n] (one scale per row) or
    [n, 4] (group = 32).  Codes are compared with the oracle's codes taken on the GPU's scales (so that
    a scale one ulp off is judged on its own), and with the oracle's own codes.  A differing code is
    allowed only where y / s lies inside the fp32 near-tie band (oracle.fp32_decision_width) and only
    by one step; the rate of differences is capped separately.
    """
    x = oracle.bf16_to_f64(x_bits)
    n = x.shape[0]
    if group == 128:
        codes_o, s_o, y = oracle.quantize_rows(x)
    else:
        codes_o, s_o, y = oracle.quantize_rows_grouped(x, group)
    sg = np.asarray(scale_bits_gpu, dtype=np.uint16).reshape(s_o.shape)
    yg = y.reshape(-1, group)
    sg_flat = sg.reshape(-1)
    at_gpu = oracle.codes_for_scales(yg, sg_flat).reshape(n, 128)
    ties = oracle.near_ties(yg, sg_flat, oracle.fp32_decision_width(x, sg, group).reshape(-1, group)).reshape(n, 128)
    got = np.asarray(codes_gpu).astype(np.int64)
    d_same = got - at_gpu
    d_own = got - codes_o
    off = d_same != 0
    return {
        "rows": n,
        "scale_max_ulp": int(np.abs(sg.astype(np.int64) - s_o.astype(np.int64)).max()) if n else 0,
        "scale_rows_differ": int(np.count_nonzero(sg != s_o)),
        "code_mismatch_frac": float(np.count_nonzero(d_own) / max(d_own.size, 1)),
        "code_mismatch_same_scale": int(np.count_nonzero(off)),
        "code_mismatch_same_scale_frac": float(np.count_nonzero(off) / max(off.size, 1)),
        "code_max_diff_same_scale": int(np.abs(d_same).max()) if d_same.size else 0,
        "code_mismatch_off_tie": int(np.count_nonzero(off & ~ties)),
        "near_tie_frac": float(ties.mean()) if ties.size else 0.0,
    }


def assert_quantize_ok(rep: dict):
    assert rep["scale_max_ulp"] <= 1, rep
    assert rep["code_mismatch_off_tie"] == 0, rep  # every differing code sits at a near-tie
    assert rep["code_max_diff_same_scale"] <= 1, rep
    assert rep["code_mismatch_same_scale_frac"] <= CODE_MISMATCH, rep
    assert rep["code_mismatch_frac"] <= CODE_MISMATCH, rep


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
