"""Pins of the oracle's kvi8r quantisation (CPU only).

Closed forms (tests/golden/kvi8r_closed_forms.json), the half-step error bound,
the absmax code, odd symmetry, power-of-two scaling and a brute-force nearest
search over the 255-point grid.  Source: "H3 Streamed Blocks" node page, Inputs
table, kv_store row; "Low VRAM, low RAM" page, "The K/V store options".
"""
import json
import os

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "kvi8r_closed_forms.json")


def _golden(name):
    with open(GOLDEN) as f:
        return next(c for c in json.load(f)["cases"] if c["name"] == name)


def _rows(name="outlier16k", tensor="k", n=4096, head=0):
    w = synth.WORKLOADS[name]
    return oracle.bf16_to_f64(synth.head_bf16(w, tensor, head)[:n])


def test_closed_form_one_hot():
    want_s = int(_golden("one_hot_unit")["scale_bits"], 16)
    h = oracle.sylvester_hadamard()
    for j in (0, 1, 77, 127):
        x = np.zeros((1, 128))
        x[0, j] = 1.0
        codes, s, _ = oracle.quantize_rows(x)
        assert s[0] == want_s
        assert np.array_equal(codes[0].astype(np.int64), 127 * h[j])


def test_closed_form_hadamard_row():
    want_s = int(_golden("hadamard_row")["scale_bits"], 16)
    h = oracle.sylvester_hadamard()
    for i in (0, 5, 64, 127):
        codes, s, _ = oracle.quantize_rows(h[i:i + 1].astype(np.float64))
        assert s[0] == want_s
        want = np.zeros(128, dtype=np.int8)
        want[i] = 127
        assert np.array_equal(codes[0], want)


def test_closed_form_zero_row():
    codes, s, _ = oracle.quantize_rows(np.zeros((3, 128)))
    assert s.tolist() == [int(_golden("zero_row")["scale_bits"], 16)] * 3
    assert not codes.any()


def test_closed_form_saturated():
    x = np.zeros((1, 128))
    x[0, 0] = 2.0 ** 30
    codes, s, _ = oracle.quantize_rows(x)
    assert s[0] == int(_golden("saturated")["scale_bits"], 16)
    assert np.all(codes == 127)


@pytest.mark.parametrize("name,tensor", [("tiny", "k"), ("outlier16k", "k"), ("outlier16k", "v")])
def test_half_step_bound_and_absmax_code(name, tensor):
    x = _rows(name, tensor)
    codes, s_bits, y = oracle.quantize_rows(x)
    s = oracle.f16_to_f64(s_bits)[:, None]
    # the fp32 decision may move a value sitting on a tie by at most a few fp32 ulps
    err = np.abs(y - codes * s)
    assert np.all(err <= s * (0.5 + 2.0 ** -14))
    arg = np.abs(y).argmax(axis=1)
    assert np.all(np.abs(codes[np.arange(len(x)), arg].astype(int)) == 127)
    assert codes.min() >= -127
    # the dequantised row is close to the rotated row (relative)
    rel = np.linalg.norm(y - codes * s) / np.linalg.norm(y)
    assert rel < 1e-2


def test_odd_symmetry():
    x = _rows()
    c1, s1, _ = oracle.quantize_rows(x)
    c2, s2, _ = oracle.quantize_rows(-x)
    assert np.array_equal(s1, s2)
    assert np.array_equal(c1.astype(int), -c2.astype(int))


@pytest.mark.parametrize("k", [-3, -1, 1, 3])
def test_power_of_two_scaling(k):
    x = _rows(n=2048)
    c1, s1, _ = oracle.quantize_rows(x)
    c2, s2, _ = oracle.quantize_rows(x * 2.0 ** k)
    assert np.array_equal(c1, c2)
    assert np.array_equal(oracle.f16_to_f64(s2), oracle.f16_to_f64(s1) * 2.0 ** k)


def test_codes_are_grid_nearest_bruteforce():
    x = _rows(n=512)
    y = oracle.rotate_rows(x)
    s_bits = oracle.row_scales(y)
    codes = oracle.codes_for_scales(y, s_bits)
    # fp32 decision variable, then nearest of the 255 grid points (ties -> even)
    v = y.astype(np.float32) / oracle.f16_to_f64(s_bits).astype(np.float32)[:, None]
    grid = np.arange(-127, 128, dtype=np.float64)
    d = np.abs(v.astype(np.float64)[..., None] - grid)
    best = d.min(axis=-1, keepdims=True)
    cand = d == best
    # among equidistant candidates the even one wins
    even_pref = np.where(cand & (grid % 2 == 0), 1, 0) + cand
    pick = grid[np.argmax(even_pref, axis=-1)]
    assert np.array_equal(codes.astype(np.float64), pick)


def test_scale_is_rounded_absmax_over_127():
    x = _rows(n=2048)
    y = x @ oracle.orthonormal_hadamard()
    a = np.abs(y).max(axis=1)
    s = oracle.f16_to_f64(oracle.row_scales(y))
    # s is one of the two fp16 neighbours of a/127 and the nearer one
    t = a / 127
    assert np.all(np.abs(s - t) <= np.abs(t) * 2.0 ** -11)


def test_rotation_spreads_outlier_channels():
    # The rotation's purpose (page: "spreads the outlier channels ... before rounding"):
    # on outlier K, per-row int8 error in the rotated basis beats the unrotated one.
    x = _rows("outlier16k", "k", n=2048)
    codes, s_bits, y = oracle.quantize_rows(x)
    rot_err = np.linalg.norm(y - oracle.dequantize_rows(codes, s_bits)) / np.linalg.norm(y)
    a = np.abs(x).max(axis=1, keepdims=True) / 127
    plain = np.clip(np.rint(x / a), -127, 127) * a
    plain_err = np.linalg.norm(x - plain) / np.linalg.norm(x)
    assert rot_err < 0.5 * plain_err


def test_chunked_build_equals_one_shot():
    x = _rows(n=1000)
    c_all, s_all, _ = oracle.quantize_rows(x)
    parts = [oracle.quantize_rows(x[i:i + 137]) for i in range(0, 1000, 137)]
    assert np.array_equal(np.concatenate([p[0] for p in parts]), c_all)
    assert np.array_equal(np.concatenate([p[1] for p in parts]), s_all)


def test_saturated_negative_clamps_to_minus_127():
    # The grid is symmetric: codes never reach -128, even when the scale saturates.
    x = np.zeros((1, 128))
    x[0, 0] = -(2.0 ** 30)
    codes, s, _ = oracle.quantize_rows(x)
    assert s[0] == 0x7BFF
    assert np.all(codes == -127)
