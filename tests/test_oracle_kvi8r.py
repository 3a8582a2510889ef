"""Pins of the oracle's kvi8r quantisation (CPU only).

Closed forms (tests/golden/kvi8r_closed_forms.json), the half-step error bound,
the absmax code, odd symmetry, power-of-two scaling, a brute-force nearest
search over the 255-point grid on the fp64 rotated values, the half-to-even
rule on exact ties, and the near-tie band: it must cover every difference an
fp32 evaluation of the code variable makes (checked against an fp32 butterfly
simulation written here) and stay narrow.  Source: "H3 Streamed Blocks" node
page, Inputs table, kv_store row; "Low VRAM, low RAM" page, "The K/V store
options".
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
    err = np.abs(y - codes * s)
    assert np.all(err <= s * 0.5)
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
    # Search the 255-point grid {c * s} for the point nearest to each fp64 rotated value; no quotient is formed.
    x = _rows(n=512)
    y = x @ oracle.orthonormal_hadamard()
    s_bits = oracle.row_scales(y)
    codes = oracle.codes_for_scales(y, s_bits)
    s = oracle.f16_to_f64(s_bits)
    grid = np.arange(-127, 128, dtype=np.float64)
    d = np.abs(y[..., None] - grid * s[:, None, None])       # |y - c s|, c s exact in fp64
    best = d.min(axis=-1)
    got = np.take_along_axis(d, (codes.astype(np.int64) + 127)[..., None], axis=-1)[..., 0]
    assert np.all(got <= best)
    # where two grid points are equally near, the even code is the one taken
    two = np.count_nonzero(d == best[..., None], axis=-1) == 2
    assert np.all(codes[two] % 2 == 0)


def test_exact_ties_round_half_to_even():
    s_bits = np.array([0x3C00, 0x2DB4], dtype=np.uint16)  # 1.0 and the Hadamard-row scale
    s = oracle.f16_to_f64(s_bits)[:, None]
    halves = np.array([0.5, 1.5, 2.5, 62.5, 63.5, 126.5, -0.5, -1.5, -125.5, 127.5, -127.5, 200.0])
    y = halves[None, :] * s  # exact in fp64: an fp16 scale times a half-integer below 2^9
    want = np.array([0, 2, 2, 62, 64, 126, 0, -2, -126, 127, -127, 127])
    assert np.array_equal(oracle.codes_for_scales(y, s_bits), np.broadcast_to(want, y.shape).astype(np.int8))
    flags = oracle.near_ties(y, s_bits, 0.0)
    assert np.array_equal(flags[0], halves != 200.0)


def test_near_tie_band_edges():
    s_bits = np.array([0x3C00], dtype=np.uint16)
    w = 2.0 ** -13  # every value below is exact in fp64
    v = np.array([[3.5, 3.5 + w, 3.5 - w, 3.5 + 2 * w, 3.5 - 2 * w, 3.0, -7.5 + 0.5 * w, -7.5 - 3 * w]])
    assert oracle.near_ties(v, s_bits, w)[0].tolist() == [True, True, True, False, False, False, True, False]
    # a zero scale means a zero row: no ties
    assert not oracle.near_ties(np.zeros((1, 4)), np.zeros(1, dtype=np.uint16), 1.0).any()


def _fp32_code_variable(x):
    """Independent fp32 evaluation of y/s: Sylvester butterflies with every add rounded to fp32, in the
    recursive order (first half / second half), then the product with the fp32 reciprocal of s*sqrt(128)."""
    z = np.asarray(x, dtype=np.float32).copy()
    h = 1
    n = z.shape[1]
    while h < n:
        z = z.reshape(z.shape[0], n // (2 * h), 2, h)
        a, b = z[:, :, 0, :].copy(), z[:, :, 1, :].copy()
        z[:, :, 0, :] = a + b
        z[:, :, 1, :] = a - b
        z = z.reshape(-1, n)
        h *= 2
    y = np.asarray(x, np.float64) @ oracle.orthonormal_hadamard()
    s_bits = oracle.row_scales(y)
    s = oracle.f16_to_f64(s_bits)
    r = np.float32(1.0) / (s * np.sqrt(128.0)).astype(np.float64)
    r32 = r.astype(np.float32).astype(np.float64)
    return z.astype(np.float64) * r32[:, None], y, s_bits


@pytest.mark.parametrize("kind", ["gauss", "outlier", "wide_range"])
def test_decision_width_covers_an_fp32_evaluation(kind):
    rng = np.random.default_rng(11)
    if kind == "wide_range":  # one large value over many tiny ones: the rounding of the large partial sums dominates
        x = rng.standard_normal((2048, 128)) * 2.0 ** rng.integers(-20, 1, size=(2048, 128))
        x[:, 0] = rng.choice([-1, 1], 2048) * 3.0e3
    else:
        x = _rows("outlier16k" if kind == "outlier" else "tiny", "k", n=2048)
    x = oracle.bf16_to_f64(synth.bf16_bits_from_f32(np.asarray(x, np.float32)))
    v32, y, s_bits = _fp32_code_variable(x)
    width = oracle.fp32_decision_width(x, s_bits)
    v = y / oracle.f16_to_f64(s_bits)[:, None]
    err = np.abs(v32 - v)
    assert np.all(err <= width)
    # the band is a bound, not a guess: it stays within a modest factor of the errors actually seen
    assert width.max() < 4e-4 and np.median(width) > np.median(err)


def test_near_ties_are_rare_on_the_workloads():
    x = _rows("outlier16k", "k", n=4096)
    codes, s_bits, y = oracle.quantize_rows(x)
    frac = oracle.near_ties(y, s_bits, oracle.fp32_decision_width(x, s_bits)).mean()
    assert 0 < frac < 1e-3


def test_scale_is_rounded_absmax_over_127():
    x = _rows(n=2048)
    y = x @ oracle.orthonormal_hadamard()
    a = np.abs(y).max(axis=1)
    s = oracle.f16_to_f64(oracle.row_scales(y))
    # s is one of the two fp16 neighbours of a/127 and the nearer one
    t = a / 127
    assert np.all(np.abs(s - t) <= np.abs(t) * 2.0 ** -11)


def test_rotation_spreads_outlier_channels():
    # What the rotation is for ("Low VRAM, low RAM" page, "The K/V store options"): it mixes the few
    # large channels into all 128 before the int8 rounding, so one outlier no longer sets the row's scale.
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
