"""Pins of the oracle's Hadamard basis and rotation invariance (CPU only).

The basis must be a fixed orthonormal 128-wide Hadamard ("H3 Streamed Blocks"
node page, Inputs table, kv_store row) and scores must be invariant under it
("Low VRAM, low RAM" page, "The K/V store options", rotation paragraph).
"""
import numpy as np
import pytest
import scipy.linalg

import oracle
import synth


def test_sylvester_is_hadamard_and_symmetric():
    h = oracle.sylvester_hadamard(128)
    assert h.shape == (128, 128)
    assert set(np.unique(h)) == {-1, 1}
    assert np.array_equal(h, h.T)
    assert np.array_equal(h @ h.T, 128 * np.eye(128, dtype=np.int64))


def test_sylvester_matches_bit_formula_and_library():
    # Independent characterisations: entry (i, j) = (-1)^popcount(i & j), and SciPy's routine.
    h = oracle.sylvester_hadamard(128)
    i, j = np.meshgrid(np.arange(128), np.arange(128), indexing="ij")
    pc = np.vectorize(lambda t: bin(int(t)).count("1"))(i & j)
    assert np.array_equal(h, np.where(pc % 2 == 0, 1, -1))
    assert np.array_equal(h, scipy.linalg.hadamard(128))


@pytest.mark.parametrize("n", [1, 2, 4, 64, 128])
def test_small_orders(n):
    h = oracle.sylvester_hadamard(n)
    assert np.array_equal(h @ h.T, n * np.eye(n, dtype=np.int64))


def test_non_power_of_two_rejected():
    with pytest.raises(ValueError):
        oracle.sylvester_hadamard(96)


def test_orthonormal_is_involution():
    hh = oracle.orthonormal_hadamard()
    assert np.abs(hh @ hh - np.eye(128)).max() < 1e-14
    assert np.abs(hh @ hh.T - np.eye(128)).max() < 1e-14


@pytest.mark.parametrize("outliers", [False, True])
def test_scores_invariant_under_rotation(outliers):
    w = synth.WORKLOADS["outlier16k" if outliers else "tiny"]
    q = oracle.bf16_to_f64(synth.head_bf16(w, "q", 0)[:200])
    k = oracle.bf16_to_f64(synth.head_bf16(w, "k", 0)[:300])
    hh = oracle.orthonormal_hadamard()
    s0 = q @ k.T
    s1 = (q @ hh) @ (k @ hh).T
    assert np.abs(s1 - s0).max() <= 1e-13 * np.abs(s0).max()
