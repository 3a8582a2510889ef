"""Pins of the per-row store routing oracle ("H3 Streamed Blocks" node page,
Inputs table, exact_av_rows row: chosen query rows attend a bf16 K/V exactly,
the others the quantised store).

Pinned on what the definition fixes: span membership against brute force, the
two degenerate routings (no span: the kvi8r path; one span over every row: the
exact path), exact rows equal to PyTorch's fp64 scaled-dot-product attention,
and a store whose quantisation error is large enough that a swapped selection
would show.
"""
import numpy as np
import pytest
import torch

import oracle
import synth

SCALE = 1.0 / np.sqrt(128)


def _case(seed, n=150, m=200, outliers=False):
    rng = np.random.default_rng(seed)
    q, k, v = (rng.standard_normal((r, 128)).astype(np.float32) for r in (n, m, m))
    if outliers:
        k[:, 5] *= 40.0  # large absmax: the kvi8r store loses most of the other channels' resolution
    qb, kb, vb = (synth.bf16_bits_from_f32(a) for a in (q, k, v))
    kc, ks, _ = oracle.quantize_rows(oracle.bf16_to_f64(kb))
    vc, vs, _ = oracle.quantize_rows(oracle.bf16_to_f64(vb))
    return qb, kb, vb, kc, ks, vc, vs


def test_spans_to_rows_brute_force():
    rng = np.random.default_rng(3)
    for _ in range(50):
        n = int(rng.integers(0, 40))
        cuts = np.sort(rng.integers(0, n + 1, size=2 * int(rng.integers(0, 4))))
        spans = cuts.reshape(-1, 2)
        got = oracle.spans_to_rows(spans, n)
        want = np.array([any(b <= i < e for b, e in spans) for i in range(n)], dtype=bool)
        assert np.array_equal(got, want)


@pytest.mark.parametrize("spans", [[(5, 3)], [(0, 4), (2, 6)], [(3, 11)], [(-1, 2)]])
def test_spans_to_rows_rejects_bad_spans(spans):
    with pytest.raises(ValueError):
        oracle.spans_to_rows(spans, 10)


def test_no_span_is_kvi8r_and_full_span_is_exact():
    qb, kb, vb, kc, ks, vc, vs = _case(1)
    n = qb.shape[0]
    none = oracle.routed_attention(qb, kb, vb, kc, ks, vc, vs, SCALE, oracle.spans_to_rows([], n))
    full = oracle.routed_attention(qb, kb, vb, kc, ks, vc, vs, SCALE, oracle.spans_to_rows([(0, n)], n))
    np.testing.assert_array_equal(none, oracle.kvi8r_attention(oracle.bf16_to_f64(qb), kc, ks, vc, vs, SCALE))
    np.testing.assert_array_equal(full, oracle.exact_attention_bf16(qb, kb, vb, SCALE))


def test_routed_rows_follow_their_store():
    qb, kb, vb, kc, ks, vc, vs = _case(2, outliers=True)
    n = qb.shape[0]
    rows = oracle.spans_to_rows([(0, 17), (64, 65), (140, 150)], n)
    got = oracle.routed_attention(qb, kb, vb, kc, ks, vc, vs, SCALE, rows)
    # exact rows: PyTorch's fp64 attention on the bf16 values
    t = [torch.from_numpy(oracle.bf16_to_f64(b))[None] for b in (qb, kb, vb)]
    sdpa = torch.nn.functional.scaled_dot_product_attention(*t, scale=SCALE)[0].numpy()
    np.testing.assert_allclose(got[rows], sdpa[rows], rtol=1e-10, atol=1e-12)
    # other rows: the kvi8r store, which differs visibly from exact attention here
    kv = oracle.kvi8r_attention(oracle.bf16_to_f64(qb), kc, ks, vc, vs, SCALE)
    np.testing.assert_array_equal(got[~rows], kv[~rows])
    assert np.abs(kv[~rows] - sdpa[~rows]).max() > 1e-3
