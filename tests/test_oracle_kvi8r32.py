"""Pins of the oracle's per-32-value kvi8r variant (CPU only).

"Low VRAM, low RAM" page, "What is next": a kvi8r variant with one scale per 32
values, finer than per row.  Reading: the rotated row is cut into four groups of
32 consecutive values, each quantised as a row of the per-row store.  Pinned on
a closed form with exactly representable scales, the per-group half-step bound
and absmax code, a brute-force nearest search, the reduction to the per-row
quantiser at one group per row, and the fact that finer scales never lose
accuracy against the per-row store.
"""
import numpy as np
import pytest

import oracle
import synth


def _rows(name="outlier16k", tensor="k", n=2048, head=0):
    w = synth.WORKLOADS[name]
    return oracle.bf16_to_f64(synth.head_bf16(w, tensor, head)[:n])


def test_closed_form_one_spike_per_group():
    # Rotated row with one spike per group, of magnitude 127 * 2^k: every scale is exactly 2^k.
    ks = [0, -1, 2, -3]
    pos = [3, 40, 64 + 17, 127]
    sign = [1, -1, 1, -1]
    y = np.zeros((1, 128))
    for k, p, sg in zip(ks, pos, sign):
        y[0, p] = sg * 127.0 * 2.0 ** k
    x = y @ oracle.orthonormal_hadamard()  # H is symmetric and orthonormal: rotating x gives back y
    codes, s, _ = oracle.quantize_rows_grouped(x)
    assert s.shape == (1, 4)
    assert s[0].tolist() == [(k + 15) << 10 for k in ks]  # fp16 bit patterns of 2^k
    want = np.zeros(128, dtype=np.int8)
    for p, sg in zip(pos, sign):
        want[p] = 127 * sg
    assert np.array_equal(codes[0], want)


@pytest.mark.parametrize("name,tensor", [("outlier16k", "k"), ("outlier16k", "v"), ("tiny", "k")])
def test_half_step_bound_and_absmax_code_per_group(name, tensor):
    codes, s, y = oracle.quantize_rows_grouped(_rows(name, tensor))
    sf = oracle.f16_to_f64(s)                       # [n, 4]
    yg = y.reshape(-1, 4, 32)
    cg = codes.astype(np.float64).reshape(-1, 4, 32)
    assert np.all(np.abs(yg - cg * sf[:, :, None]) <= sf[:, :, None] * 0.5)
    am = np.abs(yg).argmax(axis=2)
    top = np.take_along_axis(np.abs(cg), am[:, :, None], axis=2)[:, :, 0]
    assert np.all(top[sf > 0] == 127)


def test_one_group_per_row_is_the_per_row_quantiser():
    x = _rows(n=512)
    c1, s1, _ = oracle.quantize_rows(x)
    c2, s2, _ = oracle.quantize_rows_grouped(x, group=128)
    assert np.array_equal(c1, c2) and np.array_equal(s1, s2[:, 0])


def test_codes_are_grid_nearest_bruteforce():
    codes, s, y = oracle.quantize_rows_grouped(_rows(n=16))
    sf = oracle.f16_to_f64(s)
    grid = np.arange(-127, 128, dtype=np.float64)
    for i in range(y.shape[0]):
        for g in range(4):
            yy = y[i, 32 * g:32 * g + 32]
            err = np.abs(yy[:, None] - grid[None, :] * sf[i, g])
            best = err.min(axis=1)
            got = np.abs(yy - codes[i, 32 * g:32 * g + 32] * sf[i, g])
            assert np.all(got <= best)


def test_decision_width_per_group_follows_the_group_scale():
    # With four scales per row, each value's band is the per-row band taken with its own group's scale.
    x = _rows(n=1024)
    codes, s, y = oracle.quantize_rows_grouped(x)
    w4 = oracle.fp32_decision_width(x, s, group=32)
    for g in range(4):
        w_g = oracle.fp32_decision_width(x, s[:, g], group=128)
        assert np.array_equal(w4[:, 32 * g:32 * g + 32], w_g[:, 32 * g:32 * g + 32])
    assert not np.array_equal(w4[:, :32], oracle.fp32_decision_width(x, s[:, 1], group=128)[:, :32])


def test_finer_scales_never_lose_accuracy():
    x = _rows(n=2048)
    c1, s1, y = oracle.quantize_rows(x)
    c4, s4, _ = oracle.quantize_rows_grouped(x)
    e1 = y - oracle.dequantize_rows(c1, s1)
    e4 = y - oracle.dequantize_rows_grouped(c4, s4)
    row_scale = oracle.f16_to_f64(s1)[:, None]
    assert np.all(np.abs(e4) <= row_scale * 0.5)
    assert np.sum(e4 ** 2) < 0.9 * np.sum(e1 ** 2)


def test_grouped_dequantise_and_attention_reduce_to_per_row():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((300, 128))
    c, s, _ = oracle.quantize_rows(x)
    s4 = np.repeat(s[:, None], 4, axis=1)  # four equal group scales = the row scale
    assert np.array_equal(oracle.dequantize_rows_grouped(c, s4), oracle.dequantize_rows(c, s))
    q = rng.standard_normal((40, 128))
    a1 = oracle.kvi8r_attention(q, c, s, c, s, 0.0884)
    a4 = oracle.kvi8r_attention(q, c, s4, c, s4, 0.0884)
    assert np.array_equal(a1, a4)
