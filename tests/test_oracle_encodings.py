"""Pins of exact bf16/fp16 decoding and fp16 rounding used by the oracle, and of the
input generator's bf16 rounding (CPU only)."""
import numpy as np

import oracle
import synth


def test_bf16_known_patterns():
    bits = np.array([0x3F80, 0xC000, 0x0001, 0x7F7F, 0x0000, 0x8000, 0x3E80], dtype=np.uint16)
    want = [1.0, -2.0, 2.0 ** -133, (2 - 2 ** -7) * 2.0 ** 127, 0.0, -0.0, 0.25]
    got = oracle.bf16_to_f64(bits)
    assert list(got) == want


def test_f16_known_patterns():
    bits = np.array([0x3C00, 0x0001, 0x7BFF, 0x0400, 0xBC00, 0x11B4], dtype=np.uint16)
    want = [1.0, 2.0 ** -24, 65504.0, 2.0 ** -14, -1.0, (1 + 436 / 1024) * 2.0 ** -11]
    assert list(oracle.f16_to_f64(bits)) == want


def _nearest_f16_bruteforce(x):
    grid = np.arange(0x7C00, dtype=np.uint16)
    vals = grid.view(np.float16).astype(np.float64)
    idx = np.clip(np.searchsorted(vals, x), 1, len(vals) - 1)
    lo, hi = vals[idx - 1], vals[idx]
    dlo, dhi = x - lo, hi - x
    even_lo = (grid[idx - 1] & 1) == 0
    pick_lo = (dlo < dhi) | ((dlo == dhi) & even_lo)
    out = np.where(pick_lo, grid[idx - 1], grid[idx])
    out = np.where(x == hi, grid[idx], out)
    return out.astype(np.uint16)


def test_f64_to_f16_rounding_matches_bruteforce():
    rng = np.random.default_rng(0)
    vals = np.arange(0x7C00, dtype=np.uint16).view(np.float16).astype(np.float64)
    mids = (vals[:-1] + vals[1:]) / 2
    x = np.concatenate([rng.uniform(0, 65000, 100000), np.exp(rng.uniform(-18, 11, 100000)),
                        mids, np.nextafter(mids, 0), np.nextafter(mids, np.inf)])
    x = x[(x > 0) & (x < 65504)]
    assert np.array_equal(oracle.f64_to_f16_bits(x), _nearest_f16_bruteforce(x))


def test_f64_to_f16_saturates():
    assert oracle.f64_to_f16_bits(np.array([1e6, 65519.0, -1e9])).tolist() == [0x7BFF, 0x7BFF, 0xFBFF]


def test_generator_bf16_rounding_nearest_even():
    rng = np.random.default_rng(1)
    f = np.concatenate([rng.standard_normal(100000).astype(np.float32),
                        # exact ties between two bf16 neighbours
                        (np.arange(1, 2000, dtype=np.uint32) << 16 | 0x8000).view(np.float32)])
    bits = synth.bf16_bits_from_f32(f)
    got = oracle.bf16_to_f64(bits)
    lo = (f.view(np.uint32) & np.uint32(0xFFFF0000)).view(np.float32).astype(np.float64)
    hi_bits = ((f.view(np.uint32) >> 16) + 1).astype(np.uint16)
    hi = oracle.bf16_to_f64(hi_bits)
    fx = f.astype(np.float64)
    # |lo| <= |f| < |hi| in magnitude; nearest, ties to the even pattern
    dlo, dhi = np.abs(fx - lo), np.abs(hi - fx)
    lo_bits = (f.view(np.uint32) >> 16).astype(np.uint16)
    want = np.where(dlo < dhi, lo, np.where(dhi < dlo, hi, np.where(lo_bits % 2 == 0, lo, hi)))
    assert np.array_equal(got, want)
