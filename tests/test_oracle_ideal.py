"""Pins of the ideal binary64 attention (the error reference of every head,
attention-numerics project page, first section) against closed forms and the
invariances the pages state."""
import numpy as np
import pytest
from scipy.linalg import hadamard


def rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def test_identical_keys_give_running_mean_of_values(orc):
    """All keys equal -> every visible weight equal -> O_i = mean(v_0..v_i)."""
    N, d = 37, 16
    q = rand((1, 1, N, d), 1)
    k = np.broadcast_to(rand((1, 1, 1, d), 2), (1, 1, N, d)).copy()
    v = rand((1, 1, N, d), 3)
    o = orc.attention_f64(q, k, v, causal=True)
    ref = np.cumsum(v[0, 0], axis=0) / np.arange(1, N + 1)[:, None]
    np.testing.assert_allclose(o[0, 0], ref, rtol=1e-13, atol=1e-13)
    o = orc.attention_f64(q, k, v, causal=False)
    np.testing.assert_allclose(o[0, 0], np.broadcast_to(v[0, 0].mean(0), (N, d)), rtol=1e-13, atol=1e-13)


def test_first_causal_row_is_first_value(orc):
    q, k, v = rand((2, 3, 9, 8), 4), rand((2, 3, 9, 8), 5), rand((2, 3, 9, 8), 6)
    o = orc.attention_f64(q, k, v, causal=True)
    assert np.array_equal(o[:, :, 0], v[:, :, 0])


def test_two_keys_sigmoid(orc):
    """Two keys: weight of key 1 is the logistic of the logit gap."""
    d = 4
    q = np.array([[[[1.0, 0, 0, 0], [0.5, 0.5, 0, 0]]]])
    k = np.array([[[[0.3, 0.1, 0, 0], [1.2, -0.4, 0, 0]]]])
    v = np.array([[[[1.0, 0, 0, 0], [0, 1.0, 0, 0]]]])
    o = orc.attention_f64(q, k, v, causal=False, softmax_scale=0.5)
    for i in range(2):
        z = 0.5 * (q[0, 0, i] @ k[0, 0].T)
        w1 = 1.0 / (1.0 + np.exp(z[0] - z[1]))
        np.testing.assert_allclose(o[0, 0, i, :2], [1 - w1, w1], rtol=1e-14)


@pytest.mark.parametrize("causal", [True, False])
def test_shared_key_vector_cancels(orc, causal):
    """Adding one vector to every key shifts all of a query's scores equally;
    exact softmax cancels it (study page, "A shared key component should
    disappear"; project page, second section)."""
    q, k, v = rand((1, 2, 40, 16), 7), rand((1, 2, 40, 16), 8), rand((1, 2, 40, 16), 9)
    u = 20.0 * rand((1, 2, 1, 16), 10)
    o1 = orc.attention_f64(q, k, v, causal=causal)
    o2 = orc.attention_f64(q, k + u, v, causal=causal)
    np.testing.assert_allclose(o2, o1, rtol=1e-10, atol=1e-10)


@pytest.mark.parametrize("causal", [True, False])
def test_mean_key_subtraction_preserves_attention(orc, causal):
    """One vector subtracted from every key leaves binary64 softmax attention
    unchanged (project page, second section; study page, mean subtraction
    before rotation)."""
    q, k, v = rand((2, 4, 33, 16), 11), rand((2, 2, 33, 16), 12), rand((2, 2, 33, 16), 13)
    o1 = orc.attention_f64(q, k, v, causal=causal)
    o2 = orc.attention_f64(q, k - k.mean(axis=2, keepdims=True), v, causal=causal)
    np.testing.assert_allclose(o2, o1, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("d", [64, 128])
def test_hadamard_rotation_preserves_attention(orc, d):
    """The random-sign Hadamard is orthogonal, so rotating Q and K (never V)
    leaves exact attention unchanged (study page, "See the vectors and the
    arithmetic")."""
    g = np.random.default_rng(d)
    s = np.where(g.random(d) < 0.5, -1.0, 1.0)
    R = hadamard(d) * s[None, :] / np.sqrt(d)
    q, k, v = rand((1, 2, 30, d), 14), rand((1, 1, 30, d), 15), rand((1, 1, 30, d), 16)
    o1 = orc.attention_f64(q, k, v, causal=True)
    o2 = orc.attention_f64(q @ R.T, k @ R.T, v, causal=True)
    np.testing.assert_allclose(o2, o1, rtol=1e-12, atol=1e-12)


def test_gqa_equals_repeated_kv(orc):
    q, k, v = rand((2, 6, 20, 8), 17), rand((2, 2, 20, 8), 18), rand((2, 2, 20, 8), 19)
    o1 = orc.attention_f64(q, k, v, causal=True)
    o2 = orc.attention_f64(q, np.repeat(k, 3, axis=1), np.repeat(v, 3, axis=1), causal=True)
    assert np.array_equal(o1, o2)


def test_key_permutation_invariance_noncausal(orc):
    q, k, v = rand((1, 1, 25, 8), 20), rand((1, 1, 25, 8), 21), rand((1, 1, 25, 8), 22)
    perm = np.random.default_rng(1).permutation(25)
    o1 = orc.attention_f64(q, k, v, causal=False)
    o2 = orc.attention_f64(q, k[:, :, perm], v[:, :, perm], causal=False)
    np.testing.assert_allclose(o2, o1, rtol=1e-13, atol=1e-13)


def test_rows_subset_matches_full(orc):
    q, k, v = rand((1, 2, 50, 8), 23), rand((1, 1, 50, 8), 24), rand((1, 1, 50, 8), 25)
    full = orc.attention_f64(q, k, v, causal=True)
    rows = np.array([0, 7, 49, 13])
    sub = orc.attention_f64(q, k, v, causal=True, rows=rows)
    assert np.array_equal(sub, full[:, :, rows])
