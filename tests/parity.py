"""Parity gates and an oracle process pool (torch-free; test infrastructure).

Tolerances stated for this path: kvi8r output against the oracle on the same
dequantised K/V, relative L2 <= 2e-3 and max abs <= 1e-2; exact path against
the unquantised inputs, relative L2 <= 4e-3; codes differ from the oracle's in
at most 1e-4 of elements, each by one step and only at a near-tie of the fp32
evaluation; scales within 1 fp16 ulp.  The attention gates hold per head and
over all compared rows together.

The workloads name oracle samples of up to 2048 query rows on every head
against up to 217088 keys; ``OraclePool`` spreads such comparisons over
processes (one head per job, single-threaded BLAS in each), each job
regenerating its head's inputs from the seeded generators and returning only
error statistics.
"""
from __future__ import annotations

import math
import multiprocessing as mp
import os
from concurrent.futures import ProcessPoolExecutor

import numpy as np

import oracle
import synth

SCALE = 1.0 / math.sqrt(128.0)
KVI8R_REL_L2 = 2e-3
KVI8R_MAX_ABS = 1e-2
EXACT_REL_L2 = 4e-3
CODE_MISMATCH = 1e-4


def rel_l2(got, ref) -> float:
    d = np.linalg.norm(np.asarray(got, np.float64) - ref)
    n = np.linalg.norm(ref)
    return float(d / n) if n > 0 else float(d)


# ---- codes and scales ---------------------------------------------------------------

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


# ---- attention ------------------------------------------------------------------------

def _head_bits(w: synth.Workload, t: str, h: int, n: int | None) -> np.ndarray:
    b = synth.head_bf16(w, t, h)
    return b if n is None else b[:n]


def reference_rows(kind: str, w: synth.Workload, h: int, rows: np.ndarray, store_h=None, mask_h=None,
                   s_kv: int | None = None) -> np.ndarray:
    """fp64 oracle output [len(rows), 128] of one head.

    kind: "exact" | "kvi8r" (hard arm with mask_h) | "sol_exact" | "sol_kvi8r" (Sol arm, mask_h required).
    store_h: (k codes, k scale bits, v codes, v scale bits) of the head, from the GPU's store, for kvi8r kinds.
    s_kv: keys used (default: the workload's sequence).
    """
    q = synth.head_bf16(w, "q", h)[rows]
    if kind in ("exact", "sol_exact"):
        k, v = _head_bits(w, "k", h, s_kv), _head_bits(w, "v", h, s_kv)
        if kind == "sol_exact":
            return oracle.exact_sol_attention_bf16(q, k, v, SCALE, rows, mask_h)
        keep = None if mask_h is None else oracle.expand_tile_mask(mask_h, rows, k.shape[0])
        return oracle.exact_attention_bf16(q, k, v, SCALE, keep)
    kc, ks, vc, vs = store_h
    qf = oracle.bf16_to_f64(q)
    if kind == "sol_kvi8r":
        return oracle.kvi8r_sol_attention(qf, kc, ks, vc, vs, SCALE, rows, mask_h)
    keep = None if mask_h is None else oracle.expand_tile_mask(mask_h, rows, kc.shape[0])
    return oracle.kvi8r_attention(qf, kc, ks, vc, vs, SCALE, keep)


def half_ulp(x: np.ndarray, mantissa_bits: int) -> np.ndarray:
    """Half an ulp of |x| in a binary format with that many stored mantissa bits (normal range)."""
    e = np.floor(np.log2(np.maximum(np.abs(x), 2.0 ** -14)))
    return 2.0 ** (e - mantissa_bits - 1)


def attention_job(spec: dict) -> dict:
    """One head: oracle rows against the GPU's rows (fp16 bits if spec["got_f16"], else bf16), error
    statistics only.  "max_abs_beyond_bf16" is the largest error left after allowing each element the
    two roundings that separate a bf16 output from the fp16 one (half an ulp of each format)."""
    ref = reference_rows(spec["kind"], spec["workload"], spec["head"], spec["rows"], spec.get("store"),
                         spec.get("mask"), spec.get("s_kv"))
    got = (oracle.f16_to_f64 if spec.get("got_f16") else oracle.bf16_to_f64)(spec["got"])
    d = got - ref
    beyond = np.abs(d) - half_ulp(ref, 7) - half_ulp(ref, 10)
    return {"head": spec["head"], "rows": len(spec["rows"]), "rel_l2": rel_l2(got, ref),
            "max_abs": float(np.abs(d).max()) if d.size else 0.0, "err2": float(np.sum(d * d)),
            "ref2": float(np.sum(ref * ref)), "max_abs_beyond_bf16": float(beyond.max()) if d.size else 0.0}


def quantize_job(spec: dict) -> dict:
    """One (tensor, head) of a store: codes and scales against the oracle."""
    w = spec["workload"]
    x = synth.head_bf16(w, spec["tensor"], spec["head"])
    rep = quantize_report(x, spec["codes"], spec["scales"], spec.get("group", 128))
    rep.update(head=spec["head"], tensor=spec["tensor"])
    return rep


def summarise(results: list, mode: str) -> dict:
    """Pooled and per-head figures of attention_job results."""
    err2 = sum(r["err2"] for r in results)
    ref2 = sum(r["ref2"] for r in results)
    worst = max(results, key=lambda r: r["rel_l2"])
    return {"mode": mode, "heads": len(results), "rows": sum(r["rows"] for r in results),
            "rel_l2": math.sqrt(err2 / ref2) if ref2 > 0 else math.sqrt(err2),
            "worst_head": worst["head"], "worst_head_rel_l2": worst["rel_l2"],
            "max_abs": max(r["max_abs"] for r in results)}


def assert_attention_ok(results: list, mode: str) -> dict:
    """The gates, per head and pooled.  mode "kvi8r_bf16": a kvi8r store's output delivered in bf16, whose
    elements may differ from the gated fp16 output by the two roundings (see attention_job)."""
    s = summarise(results, mode)
    if mode == "kvi8r_bf16":
        bad = [r for r in results if not (r["rel_l2"] <= KVI8R_REL_L2 and r["max_abs_beyond_bf16"] <= KVI8R_MAX_ABS)]
        assert not bad and s["rel_l2"] <= KVI8R_REL_L2, (s, bad)
    elif mode in ("kvi8r", "kvi8r32", "sol_kvi8r"):
        bad = [r for r in results if not (r["rel_l2"] <= KVI8R_REL_L2 and r["max_abs"] <= KVI8R_MAX_ABS)]
        assert not bad and s["rel_l2"] <= KVI8R_REL_L2 and s["max_abs"] <= KVI8R_MAX_ABS, (s, bad)
    else:
        bad = [r for r in results if not r["rel_l2"] <= EXACT_REL_L2]
        assert not bad and s["rel_l2"] <= EXACT_REL_L2, (s, bad)
    return s


def _worker_init():
    from threadpoolctl import threadpool_limits

    threadpool_limits(1)  # one BLAS thread per process: the pool supplies the parallelism


def pool_size() -> int:
    n = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    return max(1, min(16, n))


class OraclePool:
    """Spawned worker processes for oracle jobs (spawned, not forked: the parent holds a GPU context)."""

    def __init__(self, workers: int | None = None):
        self.ex = ProcessPoolExecutor(workers or pool_size(), mp_context=mp.get_context("spawn"),
                                      initializer=_worker_init)

    def map(self, fn, specs):
        return list(self.ex.map(fn, specs))

    def submit(self, fn, spec):
        return self.ex.submit(fn, spec)

    def close(self):
        self.ex.shutdown(wait=True, cancel_futures=True)
