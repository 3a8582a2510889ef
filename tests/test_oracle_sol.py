"""Pins of the dropped-tile residual (Sol arm) oracle ("H3-Optimizations" page,
Nodes, routed-geometry paragraph: rejected tiles are replaced by block-mean K
and block-sum V merged into the softmax state).

The residual has no printed worked values.  It is pinned on what the definition
fixes: a tile whose keys are all equal is reproduced exactly by its pseudo-key
(so dropping it changes nothing), keeping every tile leaves plain attention,
and the pseudo-key depends on a tile's keys only through their mean.
"""
import numpy as np
import pytest

import oracle

SCALE = 1.0 / np.sqrt(128)


def _rng(seed):
    return np.random.default_rng(seed)


def _tiled_constant_keys(rng, m, d=128, tile=64):
    """K whose rows are equal inside each 64-row tile."""
    nt = (m + tile - 1) // tile
    base = rng.standard_normal((nt, d))
    return base[np.arange(m) // tile]


@pytest.mark.parametrize("m", [64 * 5, 64 * 4 + 7])
def test_all_kept_is_plain_attention(m):
    rng = _rng(1)
    q, k, v = rng.standard_normal((130, 128)), rng.standard_normal((m, 128)), rng.standard_normal((m, 128))
    rows = np.arange(130)
    mask = np.ones((3, (m + 63) // 64), dtype=np.uint8)
    got = oracle.sol_attention(q, k, v, SCALE, rows, mask)
    np.testing.assert_allclose(got, oracle.attention(q, k, v, SCALE), rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("m", [64 * 6, 64 * 5 + 13])
def test_constant_tiles_are_reproduced_exactly(m):
    """Every tile's keys are equal: dropping tiles (with their residual) equals full attention."""
    rng = _rng(2)
    k = _tiled_constant_keys(rng, m)
    q, v = rng.standard_normal((192, 128)), rng.standard_normal((m, 128))
    nt = (m + 63) // 64
    mask = (rng.random((3, nt)) < 0.4).astype(np.uint8)
    mask[1] = 0  # one q-tile keeps nothing: all of its attention goes through the residual
    got = oracle.sol_attention(q, k, v, SCALE, np.arange(192), mask)
    np.testing.assert_allclose(got, oracle.attention(q, k, v, SCALE), rtol=1e-11, atol=1e-12)


def test_residual_sees_only_the_tile_mean():
    """Changing a dropped tile's keys without changing their mean leaves the output unchanged,
    and changing the mean does change it."""
    rng = _rng(3)
    m = 64 * 4
    q, k, v = rng.standard_normal((64, 128)), rng.standard_normal((m, 128)), rng.standard_normal((m, 128))
    mask = np.array([[1, 0, 1, 0]], dtype=np.uint8)
    base = oracle.sol_attention(q, k, v, SCALE, np.arange(64), mask)
    d = rng.standard_normal((64, 128))
    d -= d.mean(axis=0)  # zero-mean perturbation of dropped tile 1
    k2 = k.copy()
    k2[64:128] += d
    np.testing.assert_allclose(oracle.sol_attention(q, k2, v, SCALE, np.arange(64), mask), base,
                               rtol=1e-12, atol=1e-13)
    k3 = k.copy()
    k3[64:128] += 0.5
    assert np.abs(oracle.sol_attention(q, k3, v, SCALE, np.arange(64), mask) - base).max() > 1e-3
    # and the kept tile 0 is used key by key: a zero-mean change there does change the output
    k4 = k.copy()
    k4[0:64] += d
    assert np.abs(oracle.sol_attention(q, k4, v, SCALE, np.arange(64), mask) - base).max() > 1e-3


def test_partial_tile_counts_its_real_keys():
    """A dropped partial tile of n equal keys weighs n, exactly as its n keys would."""
    rng = _rng(4)
    m = 64 * 2 + 5
    k = rng.standard_normal((m, 128))
    k[128:] = k[128]  # the 5-key partial tile has equal keys
    q, v = rng.standard_normal((64, 128)), rng.standard_normal((m, 128))
    mask = np.array([[1, 1, 0]], dtype=np.uint8)
    got = oracle.sol_attention(q, k, v, SCALE, np.arange(64), mask)
    np.testing.assert_allclose(got, oracle.attention(q, k, v, SCALE), rtol=1e-11, atol=1e-12)


def test_tile_summaries():
    rng = _rng(5)
    k, v = rng.standard_normal((64 * 2 + 3, 128)), rng.standard_normal((64 * 2 + 3, 128))
    kb, vb, n = oracle.tile_summaries(k, v)
    np.testing.assert_array_equal(n, [64, 64, 3])
    np.testing.assert_allclose(kb[2], k[128:].mean(axis=0))
    np.testing.assert_allclose(vb[1] * 64, v[64:128].sum(axis=0))


def test_kvi8r_sol_constant_tiles():
    """kvi8r store: with equal (rotated, dequantised) keys per tile, the residual equals full kvi8r attention."""
    rng = _rng(6)
    m = 64 * 3
    codes_k = np.repeat(rng.integers(-127, 128, size=(3, 128)).astype(np.int8), 64, axis=0)
    sk = np.full(m, 0x2000, dtype=np.uint16)  # fp16 scale 2^-7
    codes_v = rng.integers(-127, 128, size=(m, 128)).astype(np.int8)
    sv = np.full(m, 0x2400, dtype=np.uint16)
    q = rng.standard_normal((64, 128))
    mask = np.array([[0, 1, 0]], dtype=np.uint8)
    got = oracle.kvi8r_sol_attention(q, codes_k, sk, codes_v, sv, SCALE, np.arange(64), mask)
    full = oracle.kvi8r_attention(q, codes_k, sk, codes_v, sv, SCALE)
    np.testing.assert_allclose(got, full, rtol=1e-11, atol=1e-12)
