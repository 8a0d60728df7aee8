"""Pins of the oracle's random-sign Hadamard rotation (attention-numerics
study page: a fixed random-sign Hadamard applied to Q and K; the transform is
orthogonal, so it preserves dot products)."""
import numpy as np
import pytest
from scipy.linalg import hadamard


@pytest.mark.parametrize("d", [8, 64, 128])
def test_fwht_matches_sylvester_matrix_on_integers(orc, d):
    g = np.random.default_rng(d)
    s = np.where(g.random(d) < 0.5, -1, 1).astype(np.int8)
    x = g.integers(-50, 50, (20, d)).astype(np.float32)
    got = orc.fwht_rows(x, s)
    ref = (hadamard(d) @ (x * s).T).T        # small integers: exact
    assert np.array_equal(got, ref.astype(np.float32))


@pytest.mark.parametrize("d", [64, 128])
def test_hadamard_rows_orthogonal(orc, d):
    s = np.ones(d, np.int8)
    Hm = orc.fwht_rows(np.eye(d, dtype=np.float32), s)
    assert np.array_equal(Hm @ Hm.T, d * np.eye(d, dtype=np.float32))


@pytest.mark.parametrize("d", [64, 128])
def test_rotation_preserves_dot_products(orc, d):
    g = np.random.default_rng(3)
    s = np.where(g.random(d) < 0.5, -1, 1).astype(np.int8)
    q = g.standard_normal((50, d)).astype(np.float32)
    k = g.standard_normal((60, d)).astype(np.float32)
    rq = orc.fwht_rows(q, s).astype(np.float64)
    rk = orc.fwht_rows(k, s).astype(np.float64)
    ref = q.astype(np.float64) @ k.astype(np.float64).T
    np.testing.assert_allclose(rq @ rk.T / d, ref, atol=2e-5 * np.sqrt(d))
