"""fp64 CPU oracle for rotated-int8 ("kvi8r") K/V quantisation and chunked attention.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call, link or
run anything in this package: only the tests, the package smoke check and the
bench's CPU-baseline leg use it.  It shares no code with the HIP kernels or the
C-ABI library and imports nothing from them.

It is plain and slow on purpose: explicit matrices instead of butterflies,
fp64 NumPy throughout, per-head processing.  What it follows:

* "H3 Streamed Blocks (exact low-VRAM, alpha)" node page, Inputs table,
  kv_store row (the kvi8r store: a Hadamard rotation of each K/V row, int8
  codes, an fp16 scale per row, dequantisation per block, blockwise attention
  with a softmax combine across blocks, the query rotated in and the output
  rotated out) and q_chunk row (the result does not depend on the chunking).
* "Low VRAM, low RAM: the de-rope on a 16 GB card" page, "The K/V store
  options" (why rotating both sides leaves the scores unchanged, and the fp16
  precision inside kvi8r) and "What is next" (the one-scale-per-32-values
  variant).
* "H3-Optimizations" page, Nodes (H3 Sparse Attention and the routed-geometry
  paragraph): 64Q x 64KV tiles, a hard arm that leaves rejected tiles out and a
  Sol arm that summarises them.
* Node page, Inputs table, exact_av_rows row: a per-row choice between exact
  attention over a bf16 K/V and the quantised store.

Modules: ``hadamard`` (the basis), ``encodings`` (exact bf16/fp16 decoding and
fp16 rounding), ``kvi8r`` (quantise / dequantise), ``attention`` (exact, kvi8r,
tile-masked and blockwise log-sum-exp attention), ``sol`` (tile-masked
attention with the dropped tiles' block-mean residual), ``routing`` (per-row
choice between the exact and the kvi8r store).

Parity status: every function here is pinned by ``tests/test_oracle_*.py``
against closed forms, invariants, brute force and an independent library
routine; none is "parity unpinned".
"""
from .hadamard import sylvester_hadamard, orthonormal_hadamard
from .encodings import bf16_to_f64, f16_to_f64, f64_to_f16_bits
from .kvi8r import (rotate_rows, row_scales, codes_for_scales, fp32_decision_width, near_ties, quantize_rows,
                    dequantize_rows,
                    quantize_rows_grouped, dequantize_rows_grouped)
from .attention import (attention, attention_blockwise, kvi8r_attention, expand_tile_mask,
                        exact_attention_bf16)
from .sol import tile_summaries, sol_attention, exact_sol_attention_bf16, kvi8r_sol_attention
from .routing import spans_to_rows, routed_attention

__all__ = [
    "sylvester_hadamard", "orthonormal_hadamard", "bf16_to_f64", "f16_to_f64", "f64_to_f16_bits",
    "rotate_rows", "row_scales", "codes_for_scales", "fp32_decision_width", "near_ties", "quantize_rows",
    "dequantize_rows",
    "quantize_rows_grouped", "dequantize_rows_grouped",
    "attention", "attention_blockwise", "kvi8r_attention", "expand_tile_mask",
    "tile_summaries", "sol_attention", "exact_sol_attention_bf16", "kvi8r_sol_attention",
    "exact_attention_bf16", "spans_to_rows", "routed_attention",
]
