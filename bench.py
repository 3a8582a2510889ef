#!/usr/bin/env python3
"""Benchmark of the kvi8r / exact chunked-attention hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic input at
217088 tokens x 32 heads x 128 dims (q_chunk = kv_chunk = kv_block = 16384):
  1. build the kvi8r store: h3a_kv_quantize_pair over K and V, one call per kv_chunk;
  2. kvi8r attention: h3a_attention (rotate each query chunk, attention over the
     int8 store dequantised in the loop, un-rotate once);
  3. exact attention: h3a_attention on the bf16 store.
Inputs are resident in HBM before timing.  After the timed steps, extra legs
(each its own JSON object) time the per-row routed call (exact_av_rows), the
host-staged K/V call (store in pinned host memory, PCIe-inclusive), the
per-32-value store (kvi8r32) and one GPU's share of an 8-way head split (4 of
the 32 heads, q_chunk 16384 and 65536) at long217k, and the block-sparse path
at sparse64k: the kvi8r store's hard and Sol arms and the exact store's hard arm.
`value` is the algorithmic attention throughput of the step,
2 x 4*S*S*H*128 flop over the step's wall time.  The store build, the query
rotation and the output un-rotation are also reported as HBM rates (algorithmic
bytes per row x rows over time): kv_quantize once over its phase in the timed
step (first launch to last, gaps between launches included) and once over its
summed kernel durations, taken in separate passes after the timed steps so that
the per-launch timing events stay out of the phase; rotate_q and unrotate_o
over their kernel durations.

Prints one JSON line.  Only one GPU is supported; --gpus N with N > 1 exits.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import threading
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_FP16_TFLOPS = 2500.0  # MI355X dense fp16/bf16 matrix peak
PEAK_HBM_GBPS = 8000.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def make_inputs(w):
    import numpy as np
    import torch

    import synth

    out = {t: torch.empty((w.seq, w.heads, 128), dtype=torch.bfloat16, device="cuda") for t in ("q", "k", "v")}
    lock = threading.Lock()

    def sink(t, h, bits):
        src = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16)
        with lock:
            out[t][:, h, :].copy_(src)
            torch.cuda.synchronize()

    synth.for_each_head(w, ("q", "k", "v"), sink)
    return out


def attention_flops(w, mask=None) -> float:
    """Algorithmic flops of one attention pass: 4 * 128 per (query, kept key) pair."""
    if mask is None:
        return 4.0 * w.seq * w.seq * w.heads * 128
    import numpy as np

    t = 64
    nt = w.n_tiles
    rows = np.full(nt, t, dtype=np.float64)
    rows[-1] = w.seq - t * (nt - 1)
    keys = rows.copy()
    return float(4.0 * 128 * np.einsum("hqk,q,k->", mask.astype(np.float64), rows, keys))


KERNEL_SOURCES = ("store_kvi8r_quantize_amd/csrc/attn_fwd.hip", "store_kvi8r_quantize_amd/csrc/h3a_device.h",
                  "store_kvi8r_quantize_amd/csrc/launch.h")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_fwd_long217k_hbm_traffic.txt")


def kernel_source_digest() -> str:
    """sha256 of the attention kernel sources with comments and blank space removed, so that an edit of
    comments alone keeps the digest (and the counters taken on the code) while any code change alters it."""
    import hashlib
    import re

    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), encoding="utf-8") as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)       # block comments
        text = re.sub(r"//[^\n]*", " ", text)                    # line comments (no // inside strings here)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()


def measured_traffic(mode: str):
    """HBM bytes per launch of the attention kernel from the committed FETCH_SIZE / WRITE_SIZE summary.

    The summary records the digest of the kernel sources it was taken on
    (kernel_source_digest); if the code has changed since, the figure no longer
    describes this kernel and None is returned.
    """
    try:
        text = open(TRAFFIC_FILE).read()
    except OSError:
        return None
    digest = kernel_source_digest()
    vals = {}
    for line in text.splitlines():
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            vals[k.strip()] = v.split()[0] if v.split() else ""
    if vals.get("source_digest") != digest:
        return None
    v = vals.get(f"traffic_bytes_per_launch {mode}")
    return float(v) if v else None


def cpu_baseline(w, store, seconds: float):
    """The fp64 oracle on a bounded sample: kvi8r attention of head 0 rows against the full store."""
    import numpy as np

    import oracle
    import synth

    blas = "unknown"
    try:
        from threadpoolctl import threadpool_info

        pools = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        cores = max([i.get("num_threads", 1) for i in pools] or [1])
        if pools:
            blas = f"{pools[0].get('internal_api', '?')} {pools[0].get('version', '')}".strip()
    except Exception:  # threadpoolctl missing: report the affinity size
        cores = len(os.sched_getaffinity(0))
    kc, vc, sc = store
    host = lambda t: t.cpu().contiguous().view(__import__("torch").int16).numpy().view(np.uint16)
    kcodes, ks = kc[0].cpu().numpy(), host(sc[0, 0])
    vcodes, vs = vc[0].cpu().numpy(), host(sc[1, 0])
    q = oracle.bf16_to_f64(synth.head_bf16(w, "q", 0))
    scale = 1.0 / math.sqrt(128)
    block = 256
    rows = 0
    t0 = time.perf_counter()
    while True:
        r0 = (rows * 7919) % (w.seq - block)
        oracle.kvi8r_attention(q[r0:r0 + block], kcodes, ks, vcodes, vs, scale)
        rows += block
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    flops = 4.0 * rows * w.seq * 128
    full = 4.0 * w.seq * w.seq * w.heads * 128  # one whole kvi8r attention pass
    return {"value": flops / el / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": f"kvi8r attention (fp64 NumPy oracle) of {rows} query rows of head 0 against all "
                      f"{w.seq} keys, in blocks of {block} rows, {el:.1f} s",
            "blas": blas, "seconds_for_one_full_pass": round(full / (flops / el), 1)}


def sparse_legs(h3a, dev, reps: int):
    """Attention over the 64Q x 64KV tile-masked sparse64k workload (30 % video KV density): kvi8r
    store, hard arm (dropped tiles left out) and Sol arm (each dropped tile one pseudo-key); and the
    exact bf16 store, hard arm."""
    import numpy as np
    import torch

    import synth

    w = synth.WORKLOADS["sparse64k"]
    x = make_inputs(w)
    mask_np = synth.tile_mask(w)
    mask = torch.from_numpy(mask_np).to(dev)
    kc, vc, sc = h3a.new_kvi8r_store(w.seq, w.heads, device=dev)
    for t0 in range(0, w.seq, w.q_chunk):
        h3a.h3a_kv_quantize(x["k"][t0:t0 + w.q_chunk], kc, sc[0], token_offset=t0)
        h3a.h3a_kv_quantize(x["v"][t0:t0 + w.q_chunk], vc, sc[1], token_offset=t0)
    outs = {"kvi8r": torch.empty(x["q"].shape, dtype=torch.float16, device=dev),
            "exact": torch.empty_like(x["q"])}
    stores = {"kvi8r": (kc, vc, sc), "exact": (x["k"], x["v"], None)}
    stream = torch.cuda.current_stream(dev)
    # query rows per q-tile and pseudo-keys (dropped tiles) per (head, q-tile)
    rows = np.full(w.n_tiles, 64.0)
    rows[-1] = w.seq - 64 * (w.n_tiles - 1)
    pseudo_flops = float(4.0 * 128 * np.einsum("hq,q->", (mask_np == 0).sum(axis=2).astype(np.float64), rows))
    res = {}
    for mode, sol in (("kvi8r", False), ("kvi8r", True), ("exact", False)):
        ws = torch.empty(max(h3a.h3a_attention_workspace_bytes(w.seq, w.seq, w.heads, w.q_chunk, mode, True,
                                                               sol=sol), 256), dtype=torch.uint8, device=dev)
        call = lambda: h3a.h3a_attention(x["q"], *stores[mode], outs[mode], q_chunk=w.q_chunk, mode=mode,
                                         tile_mask=mask, sol=sol, workspace=ws)
        call()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            call()
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        flops = attention_flops(w, mask_np) + (pseudo_flops if sol else 0.0)
        tflops = flops / (ms / 1000) / 1e12
        r = {"workload": w.name, "mode": mode, "arm": "sol" if sol else "hard", "seq": w.seq, "heads": w.heads,
             "q_chunk": w.q_chunk, "kept_tile_frac": round(float(mask_np.mean()), 4),
             "tflop_algorithmic": round(flops / 1e12, 3), "ms": round(ms, 3), "tflops": round(tflops, 2),
             "frac_of_peak": round(tflops / PEAK_FP16_TFLOPS, 4)}
        if sol:
            r["pseudo_keys_per_row"] = round(float((mask_np == 0).sum(axis=2).mean()), 1)
            r["ms_over_hard"] = round(ms - res["sparse64k"]["ms"], 3)
        res["sparse64k_sol" if sol else "sparse64k" if mode == "kvi8r" else "sparse64k_exact"] = r
        del ws
    return res


def routed_leg(h3a, w, x, store, kvi8r_ms: float, ws, stream, reps: int = 2):
    """h3a_attention_routed at long217k: a 5760-row text prefix and a 2240-row audio tail (3.7 % of the
    rows, the text + audio share the node page gives) attend the bf16 K/V exactly, the rest the kvi8r store."""
    import torch

    spans = [(0, 5760), (w.seq - 2240, w.seq)]
    out = torch.empty_like(x["q"])
    call = lambda: h3a.h3a_attention_routed(x["q"], x["k"], x["v"], store, out, exact_spans=spans,
                                            q_chunk=w.q_chunk, kv_block=w.kv_block, workspace=ws)
    call()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    flops = attention_flops(w)
    return {"workload": w.name, "exact_spans": spans, "exact_row_frac": round(8000 / w.seq, 4),
            "ms": round(ms, 3), "tflops": round(flops / (ms / 1000) / 1e12, 2),
            "ms_vs_kvi8r": round(ms - kvi8r_ms, 3)}


def kvi8r32_leg(h3a, w, x, ws, stream, reps: int = 2):
    """The per-32-value store (kvi8r32) at long217k: build (h3a_kv_quantize_g32 per kv_chunk) and attention."""
    import torch

    kc, vc, sc = h3a.new_kvi8r_store(w.seq, w.heads, device=x["q"].device, per32=True)
    out = torch.empty(x["q"].shape, dtype=torch.float16, device=x["q"].device)

    def build():
        for t0 in range(0, w.seq, w.q_chunk):
            h3a.h3a_kv_quantize(x["k"][t0:t0 + w.q_chunk], kc, sc[0], token_offset=t0)
            h3a.h3a_kv_quantize(x["v"][t0:t0 + w.q_chunk], vc, sc[1], token_offset=t0)

    attend = lambda: h3a.h3a_attention(x["q"], kc, vc, sc, out, q_chunk=w.q_chunk, kv_block=w.kv_block,
                                       mode="kvi8r32", workspace=ws)
    build()
    attend()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    q_ms = a_ms = 0.0
    for _ in range(reps):
        ev[0].record(stream)
        build()
        ev[1].record(stream)
        attend()
        ev[2].record(stream)
        torch.cuda.synchronize()
        q_ms += ev[0].elapsed_time(ev[1])
        a_ms += ev[1].elapsed_time(ev[2])
    q_ms, a_ms = q_ms / reps, a_ms / reps
    flops = attention_flops(w)
    store_bytes = 2.0 * w.seq * w.heads * (256 + 128 + 8)  # per tensor row: bf16 in, int8 codes + 4 fp16 scales out
    return {"workload": w.name, "mode": "kvi8r32", "quant_ms": round(q_ms, 3),
            "quant_GB_per_s": round(store_bytes / (q_ms / 1000) / 1e9, 1), "attention_ms": round(a_ms, 3),
            "tflops": round(flops / (a_ms / 1000) / 1e12, 2),
            "frac_of_peak": round(flops / (a_ms / 1000) / 1e12 / PEAK_FP16_TFLOPS, 4)}


def host_kv_leg(h3a, w, x, store, dev_ms: dict, stream, reps: int = 1, wide_q_chunk: int = 65536):
    """h3a_attention_host_kv at long217k: the kvi8r and exact stores in pinned host memory, streamed one
    kv_block at a time per query chunk.  Reports the time against the resident store and the PCIe bytes moved,
    at the workload's q_chunk and at a wider one: the store crosses PCIe once per query chunk, and the output
    does not depend on q_chunk, so a caller with room for the wider chunk's per-row state moves fewer bytes."""
    import torch

    res = {}
    for mode in ("kvi8r", "exact"):
        if mode == "kvi8r":
            host = [torch.empty(t.shape, dtype=t.dtype, pin_memory=True).copy_(t) for t in store]
            store_bytes = sum(t.numel() * t.element_size() for t in host)
        else:
            host = [torch.empty(x[t].shape, dtype=x[t].dtype, pin_memory=True).copy_(x[t]) for t in ("k", "v")]
            host.append(None)
            store_bytes = sum(t.numel() * t.element_size() for t in host[:2])
        out = torch.empty(x["q"].shape, dtype=torch.float16 if mode == "kvi8r" else torch.bfloat16,
                          device=x["q"].device)
        for qc in (w.q_chunk, wide_q_chunk):
            need = h3a.h3a_attention_host_kv_workspace_bytes(w.seq, w.seq, w.heads, qc, w.kv_block, mode)
            ws = torch.empty(max(need, 256), dtype=torch.uint8, device=x["q"].device)
            call = lambda: h3a.h3a_attention_host_kv(x["q"], *host, out, q_chunk=qc, kv_block=w.kv_block,
                                                     mode=mode, workspace=ws)
            call()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(reps):
                call()
            e1.record(stream)
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / reps
            n_chunks = -(-w.seq // qc)
            pcie = store_bytes * n_chunks
            r = {"ms": round(ms, 3), "ms_resident": round(dev_ms[mode], 3),
                 "tflops": round(attention_flops(w) / (ms / 1000) / 1e12, 2),
                 "host_to_device_GB": round(pcie / 1e9, 2), "host_to_device_GB_per_s": round(pcie / ms / 1e6, 1),
                 "device_workspace_GB": round(need / 1e9, 3), "resident_store_GB": round(store_bytes / 1e9, 3)}
            if qc == w.q_chunk:
                res[mode] = r
            else:
                res[mode]["wide_q_chunk"] = {"q_chunk": qc, **r}
            del ws
        del host, out
    return {"workload": w.name, "kv_block": w.kv_block, "q_chunk": w.q_chunk, **res}


def shard_leg(h3a, w, x, stream, heads: int = 4, reps: int = 2):
    """One GPU's share of the workload split by heads over 8 GPUs: the same S, heads 0..3, a store built
    for them, attention at q_chunk 16384 and 65536 (the grid has one workgroup per 256 rows and head)."""
    import torch

    xs = {t: x[t][:, :heads].contiguous() for t in ("q", "k", "v")}
    kc, vc, sc = h3a.new_kvi8r_store(w.seq, heads, device=xs["q"].device)
    for t0 in range(0, w.seq, w.q_chunk):
        h3a.h3a_kv_quantize(xs["k"][t0:t0 + w.q_chunk], kc, sc[0], token_offset=t0)
        h3a.h3a_kv_quantize(xs["v"][t0:t0 + w.q_chunk], vc, sc[1], token_offset=t0)
    out_r = torch.empty(xs["q"].shape, dtype=torch.float16, device=xs["q"].device)
    out = torch.empty_like(xs["q"])
    flops = 4.0 * w.seq * w.seq * heads * 128
    res = {"workload": w.name, "seq": w.seq, "heads": heads, "share_of": f"{w.heads} heads over {w.heads // heads} GPUs"}
    for q_chunk in (w.q_chunk, 4 * w.q_chunk):
        ws_bytes = max(h3a.h3a_attention_workspace_bytes(w.seq, w.seq, heads, q_chunk, m, False)
                       for m in ("kvi8r", "exact"))
        ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=xs["q"].device)
        calls = {
            "kvi8r": lambda: h3a.h3a_attention(xs["q"], kc, vc, sc, out_r, q_chunk=q_chunk, kv_block=w.kv_block,
                                               mode="kvi8r", workspace=ws),
            "exact": lambda: h3a.h3a_attention(xs["q"], xs["k"], xs["v"], None, out, q_chunk=q_chunk,
                                               kv_block=w.kv_block, mode="exact", workspace=ws),
        }
        entry = {"workgroups_per_launch": -(-min(q_chunk, w.seq) // 256) * heads}
        for mode, call in calls.items():
            call()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(reps):
                call()
            e1.record(stream)
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / reps
            entry[mode] = {"ms": round(ms, 3), "tflops": round(flops / (ms / 1000) / 1e12, 2),
                           "frac_of_peak": round(flops / (ms / 1000) / 1e12 / PEAK_FP16_TFLOPS, 4)}
        res[f"q_chunk_{q_chunk}"] = entry
        del ws
    return res


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--workload", default="long217k")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-sparse", action="store_true", help="skip the block-sparse (sparse64k) legs")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after the timed region, run one plain 1 GiB device-to-device copy (a known-size "
                         "reference for HBM traffic counters)")
    ap.add_argument("--no-routed", action="store_true", help="skip the per-row routed (exact_av_rows) leg")
    ap.add_argument("--no-kvi8r32", action="store_true", help="skip the per-32-value store (kvi8r32) leg")
    ap.add_argument("--no-host-kv", action="store_true", help="skip the host-staged K/V leg")
    ap.add_argument("--no-shard", action="store_true",
                    help="skip the one-GPU-share leg (4 of the 32 heads, as with 8 GPUs split by heads)")
    ap.add_argument("--sparse-only", action="store_true",
                    help="run only the block-sparse legs and print their JSON (for profiling the sparse kernels)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "the path shards by heads with no exchange, see the design notes", file=sys.stderr)
        return 2

    import torch

    import store_kvi8r_quantize_amd as h3a
    import synth

    w = synth.WORKLOADS[args.workload]
    if w.sparse:
        raise SystemExit("bench.py times the dense long-sequence workload; sparse workloads are parity cases")
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.sparse_only:
        print(json.dumps(sparse_legs(h3a, dev, reps=max(args.steps, 1))), flush=True)
        return 0
    log(f"generating {w.name}: S={w.seq} H={w.heads}")
    t_gen = time.time()
    x = make_inputs(w)
    log(f"inputs resident in {time.time() - t_gen:.1f} s")
    kc, vc, sc = h3a.new_kvi8r_store(w.seq, w.heads, device=dev)
    out_r = torch.empty(x["q"].shape, dtype=torch.float16, device=dev)  # the kvi8r output is fp16 (H3A_OUT_F16)
    out_e = torch.empty_like(x["q"])
    ws_bytes = max(h3a.h3a_attention_workspace_bytes(w.seq, w.seq, w.heads, w.q_chunk, m, False)
                   for m in ("kvi8r", "exact"))
    ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    ev = {k: [torch.cuda.Event(enable_timing=True) for _ in range(2)] for k in ("quant", "kvi8r", "exact")}
    acc_ms = {k: 0.0 for k in ev}

    def step(record: bool):
        if record:
            ev["quant"][0].record(stream)
        for t0 in range(0, w.seq, w.q_chunk):  # K and V of each kv_chunk in one launch
            h3a.h3a_kv_quantize_pair(x["k"][t0:t0 + w.q_chunk], x["v"][t0:t0 + w.q_chunk], kc, vc, sc,
                                     token_offset=t0)
        if record:
            ev["quant"][1].record(stream)
            ev["kvi8r"][0].record(stream)
            h3a.h3a_timing_enable(True)  # the kvi8r pass's kernels are timed one by one; the store build is not
        h3a.h3a_attention(x["q"], kc, vc, sc, out_r, q_chunk=w.q_chunk, kv_block=w.kv_block, mode="kvi8r",
                          workspace=ws)
        if record:
            ev["kvi8r"][1].record(stream)
            ev["exact"][0].record(stream)
        h3a.h3a_timing_enable(False)
        h3a.h3a_attention(x["q"], x["k"], x["v"], None, out_e, q_chunk=w.q_chunk, kv_block=w.kv_block,
                          mode="exact", workspace=ws)
        if record:
            ev["exact"][1].record(stream)

    for i in range(args.warmup):
        step(False)
        torch.cuda.synchronize()
        log(f"warmup step {i + 1}/{args.warmup} done")

    # Timed region: K steps between two device synchronisations.  Attention-kernel
    # launches of the kvi8r pass are bracketed by library-side HIP events.
    kern_ms, kern_n = 0.0, 0
    side = {k: [0.0, 0] for k in ("rotate_q", "unrotate_o", "kv_quantize")}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(True)
        h3a.h3a_timing_enable(False)
        torch.cuda.synchronize()
        for k in ev:
            acc_ms[k] += ev[k][0].elapsed_time(ev[k][1])
        ms, n = h3a.h3a_timing_collect()
        kern_ms += ms
        kern_n += n
        for k in side:
            ms, n = h3a.h3a_timing_collect(k)
            side[k][0] += ms
            side[k][1] += n
        log(f"step {i + 1}/{args.steps}: kvi8r {ev['kvi8r'][0].elapsed_time(ev['kvi8r'][1]):.1f} ms, "
            f"exact {ev['exact'][0].elapsed_time(ev['exact'][1]):.1f} ms")
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1000.0 / args.steps
    # The store build's kernel durations, from passes of their own: the timing events around its 14
    # launches would add ~7 us each to the phase measured above.
    h3a.h3a_timing_enable(True)
    for i in range(args.steps):
        for t0_ in range(0, w.seq, w.q_chunk):
            h3a.h3a_kv_quantize_pair(x["k"][t0_:t0_ + w.q_chunk], x["v"][t0_:t0_ + w.q_chunk], kc, vc, sc,
                                     token_offset=t0_)
    h3a.h3a_timing_enable(False)
    ms, n = h3a.h3a_timing_collect("kv_quantize")
    side["kv_quantize"][0] += ms
    side["kv_quantize"][1] += n

    f_mode = attention_flops(w)
    tflops = 2 * f_mode / (ms_step / 1000.0) / 1e12
    per = {k: acc_ms[k] / args.steps for k in acc_ms}
    kern_avg_ms = kern_ms / max(kern_n, 1)
    flops_per_launch = f_mode * args.steps / max(kern_n, 1)
    achieved = flops_per_launch / (kern_avg_ms / 1000.0) / 1e12
    quant_bytes = 2.0 * w.seq * w.heads * (256 + 128 + 2)
    exps = float(w.seq) * w.seq * w.heads  # one exponential per (query, key) pair and head
    rows_per_step = float(w.seq) * w.heads  # rotated and un-rotated once per query row and head
    kq_ms = side["kv_quantize"][0]
    kq_gbs = round(quant_bytes * args.steps / (kq_ms / 1000) / 1e9, 1) if kq_ms > 0 else None
    kq_frac = round(kq_gbs / PEAK_HBM_GBPS, 4) if kq_gbs else None
    side_json = {}
    for k, per_row in (("rotate_q", 256 + 256), ("unrotate_o", 512 + 256)):
        ms_tot, n = side[k]
        gbs = rows_per_step * args.steps * per_row / (ms_tot / 1000) / 1e9 if ms_tot > 0 else None
        side_json[k] = {"ms_per_step": round(ms_tot / args.steps, 3), "launches_per_step": n // args.steps,
                        "bytes_per_row": per_row, "GB_per_s": None if gbs is None else round(gbs, 1),
                        "frac_of_hbm_peak": None if gbs is None else round(gbs / PEAK_HBM_GBPS, 4)}
    res = {
        "metric": "attention TFLOP/s at 217k tok, 32h x 128d (kvi8r/exact); % fp16 MFMA peak",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16+bf16 (fp32 accumulate)",
        "data": "synthetic",
        "config": {"workload": w.name, "seq": w.seq, "heads": w.heads, "head_dim": 128, "q_chunk": w.q_chunk,
                   "kv_chunk": w.q_chunk, "kv_block": w.kv_block, "modes": ["kvi8r", "exact"],
                   "step": "kv_quantize(K,V) + attention(kvi8r) + attention(exact)"},
        "frac_of_peak": round(tflops / PEAK_FP16_TFLOPS, 4),
        "phases_ms": {k: round(v, 3) for k, v in per.items()},
        "modes": {
            m: {"tflops": round(f_mode / (per[m] / 1000) / 1e12, 2),
                "frac_of_peak": round(f_mode / (per[m] / 1000) / 1e12 / PEAK_FP16_TFLOPS, 4),
                "exps": exps, "exps_per_s": round(exps / (per[m] / 1000), 1)}
            for m in ("kvi8r", "exact")
        },
        "kvi8r_output": "fp16 (H3A_OUT_F16)",
        **side_json,
        # phase time (first launch to last, launch gaps included) and the summed kernel durations
        "kv_quantize": {"ms": round(per["quant"], 3), "GB_per_s": round(quant_bytes / (per["quant"] / 1000) / 1e9, 1),
                        "frac_of_hbm_peak": round(quant_bytes / (per["quant"] / 1000) / 1e9 / PEAK_HBM_GBPS, 4),
                        "kernel_ms": round(side["kv_quantize"][0] / args.steps, 3),
                        "kernel_GB_per_s": kq_gbs, "kernel_frac_of_hbm_peak": kq_frac,
                        "bytes_per_row": 256 + 128 + 2,
                        "launches": side["kv_quantize"][1] // args.steps,
                        "call": "h3a_kv_quantize_pair (K and V of a chunk)"},
        "roofline": {"kernel": "attn_fwd_dense_kernel<1, false> (kvi8r, dense)", "bound": "mfma",
                     "achieved": round(achieved, 2), "peak": PEAK_FP16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_FP16_TFLOPS, 4), "traffic": measured_traffic("kvi8r"),
                     "traffic_unit": "HBM bytes per launch (FETCH_SIZE x fetch factor + WRITE_SIZE x write factor)",
                     "launches_per_step": kern_n // args.steps, "avg_launch_ms": round(kern_avg_ms, 3),
                     "flops_per_launch": flops_per_launch},
    }
    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        res["copy_calibration_bytes"] = 1 << 30
        del src, dst
    if not args.no_routed:
        log("routed leg ...")
        res["long217k_routed"] = routed_leg(h3a, w, x, (kc, vc, sc), per["kvi8r"], ws, stream)
        log(f"routed: {res['long217k_routed']['ms']} ms ({res['long217k_routed']['ms_vs_kvi8r']:+.1f} ms vs kvi8r)")
    if not args.no_host_kv:
        log("host-staged K/V leg ...")
        res["long217k_host_kv"] = host_kv_leg(h3a, w, x, (kc, vc, sc), per, stream)
        hk = res["long217k_host_kv"]
        log(f"host-staged: kvi8r {hk['kvi8r']['ms']} ms, exact {hk['exact']['ms']} ms; at q_chunk "
            f"{hk['exact']['wide_q_chunk']['q_chunk']}: kvi8r {hk['kvi8r']['wide_q_chunk']['ms']} ms, "
            f"exact {hk['exact']['wide_q_chunk']['ms']} ms")
    if not args.no_kvi8r32:
        log("kvi8r32 leg ...")
        del out_r
        res["long217k_kvi8r32"] = kvi8r32_leg(h3a, w, x, ws, stream)
        log(f"kvi8r32: attention {res['long217k_kvi8r32']['tflops']} TFLOP/s")
    if not args.no_shard:
        log("head-shard leg ...")
        res["long217k_h4_shard"] = shard_leg(h3a, w, x, stream)
        sh = res["long217k_h4_shard"]
        log("head shard (4 heads): " + ", ".join(f"{k} kvi8r {v['kvi8r']['tflops']} exact {v['exact']['tflops']}"
                                                 for k, v in sh.items() if k.startswith("q_chunk")))
    if not args.no_sparse:
        log("sparse64k leg ...")
        del x, out_e, ws
        torch.cuda.empty_cache()
        res.update(sparse_legs(h3a, dev, reps=3))
        log(f"sparse64k: hard {res['sparse64k']['tflops']} TFLOP/s, sol {res['sparse64k_sol']['tflops']} TFLOP/s, "
            f"exact store {res['sparse64k_exact']['tflops']} TFLOP/s")
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) ...")
        res["cpu_baseline"] = cpu_baseline(w, (kc, vc, sc), args.cpu_seconds)
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
