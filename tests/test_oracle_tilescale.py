"""Pins of the oracle's per-tile Q/K scaling (one max-based scale per
128-token tile instead of per (batch, head): the earlier emulator's
granularity, which the attention-numerics project page, second section,
contrasts with FA3's per-head scales).  Reading: tiles of 128 tokens, V keeps
its per-head scale, and the running max is kept in scaled units."""
import numpy as np
import pytest

import oracle
import synth

T = 128


def operands(seed, N, hq=2, hkv=1, d=64, tile_gain=None):
    g = np.random.default_rng(seed)
    q = g.standard_normal((1, hq, N, d)).astype(np.float32)
    k = g.standard_normal((1, hkv, N, d)).astype(np.float32)
    v = g.standard_normal((1, hkv, N, d)).astype(np.float32)
    if tile_gain is not None:
        for t in range((N + T - 1) // T):
            q[:, :, t * T:(t + 1) * T] *= np.float32(tile_gain[t % len(tile_gain)])
            k[:, :, t * T:(t + 1) * T] *= np.float32(tile_gain[(t + 1) % len(tile_gain)])
    return q, k, v


def signs(d):
    return np.where(np.random.default_rng(7).random(d) < 0.5, -1, 1).astype(np.int8)


@pytest.mark.parametrize("N", [1, 100, 128])
@pytest.mark.parametrize("flags", [dict(), dict(rotate=True), dict(rotate=True, center=True)])
def test_single_tile_is_the_per_head_path(N, flags):
    q, k, v = operands(1, N)
    s = signs(64) if flags.get("rotate") else None
    a = oracle.prepare(q, k, v, signs=s, **flags)
    b = oracle.prepare(q, k, v, signs=s, tiles=True, **flags)
    for x, y in ((a.q8, b.q8), (a.k8, b.k8), (a.v8, b.v8)):
        assert np.array_equal(x, y)
    assert np.array_equal(a.q_desc.ravel(), b.q_desc.ravel()) and np.array_equal(a.k_desc.ravel(), b.k_desc.ravel())
    ra = oracle.attention_fp8(a, kv_order=1, want_p=True)
    rb = oracle.attention_fp8(b, kv_order=1, want_p=True)
    assert np.array_equal(ra.out, rb.out) and np.array_equal(ra.p, rb.p)


@pytest.mark.parametrize("order", [0, 1])
@pytest.mark.parametrize("block_n", [64, 128])
@pytest.mark.parametrize("causal", [True, False])
def test_equal_tile_maxima_reduce_to_per_head(order, block_n, causal):
    """Every tile holds the same largest magnitude, so every tile scale equals
    the per-head one and the loop must give the per-head bytes."""
    N = 400
    q, k, v = operands(2, N)
    q = np.clip(q, -2.5, 2.5)
    k = np.clip(k, -2.5, 2.5)
    for t in range((N + T - 1) // T):
        q[:, :, t * T, 3] = 3.0
        k[:, :, t * T + 1, 5] = -3.0
    a = oracle.prepare(q, k, v)
    b = oracle.prepare(q, k, v, tiles=True)
    assert np.all(b.q_desc == a.q_desc[..., None]) and np.all(b.k_desc == a.k_desc[..., None])
    kw = dict(kv_order=order, block_n=block_n, causal=causal, want_p=True, k_sink=4)
    ra, rb = oracle.attention_fp8(a, **kw), oracle.attention_fp8(b, **kw)
    assert np.array_equal(ra.out, rb.out) and np.array_equal(ra.p, rb.p)
    assert np.array_equal(ra.row_zeros, rb.row_zeros)


def test_tile_scales_are_tile_maxima():
    N = 300
    q, k, v = operands(3, N, tile_gain=(1.0, 4.0, 0.25))
    p = oracle.prepare(q, k, v, tiles=True)
    for t in range(3):
        sl = slice(t * T, min((t + 1) * T, N))
        for x, desc, codes in ((q, p.q_desc, p.q8), (k, p.k_desc, p.k8)):
            A = np.abs(x[0, 0, sl]).max()
            assert desc[0, 0, t] == np.float32(np.float32(A) / np.float32(448.0))
            assert np.abs(oracle.e4m3_decode(codes[0, 0, sl])).max() == 448.0


def test_power_of_two_tile_gain_moves_only_that_tiles_descale():
    N = 384
    q, k, v = operands(4, N)
    a = oracle.prepare(q, k, v, rotate=True, signs=signs(64), tiles=True)
    q2, k2 = q.copy(), k.copy()
    q2[:, :, T:2 * T] *= np.float32(2.0 ** 5)
    k2[:, :, 2 * T:3 * T] *= np.float32(2.0 ** -3)
    b = oracle.prepare(q2, k2, v, rotate=True, signs=signs(64), tiles=True)
    assert np.array_equal(a.q8, b.q8) and np.array_equal(a.k8, b.k8)
    fq = b.q_desc / a.q_desc
    fk = b.k_desc / a.k_desc
    assert np.array_equal(fq[0, :, 1], np.full(2, 32.0, np.float32)) and np.all(np.delete(fq, 1, axis=2) == 1)
    assert np.array_equal(fk[0, :, 2], np.full(1, 0.125, np.float32)) and np.all(np.delete(fk, 2, axis=2) == 1)


@pytest.mark.parametrize("order", [0, 1])
def test_loop_matches_softmax_of_dequantised_operands(order):
    """Tiles whose magnitudes differ by up to 8x: the loop's output agrees with
    binary64 softmax attention on the dequantised codes to within P~'s
    quantisation noise; a wrong tile in the logit factor would scale logits by
    2-8x and miss by far more."""
    N, d = 512, 64
    q, k, v = operands(5, N, d=d, tile_gain=(1.0, 8.0, 0.5, 2.0))
    p = oracle.prepare(q, k, v, tiles=True)
    tq = np.repeat(p.q_desc[0, :, :], T, axis=1)[:, :N]            # [Hq, N]
    tk = np.repeat(p.k_desc[0, 0, :], T)[:N]                        # [N]
    qd = oracle.e4m3_decode(p.q8[0]).astype(np.float64) * tq[:, :, None]
    kd = oracle.e4m3_decode(p.k8[0, 0]).astype(np.float64) * tk[:, None]
    vd = oracle.e4m3_decode(p.v8[0, 0]).astype(np.float64) * float(p.v_desc[0, 0])
    z = np.einsum("hnd,md->hnm", qd, kd) * float(np.float32(1 / np.sqrt(d)))
    z = np.where(np.tril(np.ones((N, N), bool)), z, -np.inf)
    w = np.exp(z - z.max(-1, keepdims=True))
    ref = (w / w.sum(-1, keepdims=True)) @ vd
    out = oracle.attention_fp8(p, kv_order=order).out[0].astype(np.float64)
    rel = np.sqrt(((out - ref) ** 2).sum((-2, -1)) / (ref ** 2).sum((-2, -1)))
    assert rel.max() < 2e-2, rel


def test_prefix_scales_are_running_maxima_of_tile_maxima():
    """Prefix scales: tile t uses the largest tile maximum among tiles 0..t;
    where tile maxima only grow they equal the plain tile scales, and codes of
    a tile whose scale comes from an earlier tile are that tile's values at the
    earlier scale."""
    N = 640
    q, k, v = operands(6, N, tile_gain=(2.0, 0.5, 1.0, 4.0, 0.25))
    a = oracle.prepare(q, k, v, rotate=True, signs=signs(64), tiles=True)
    b = oracle.prepare(q, k, v, rotate=True, signs=signs(64), tiles=True, prefix=True)
    for x, y in ((a.q_desc, b.q_desc), (a.k_desc, b.k_desc)):
        assert np.array_equal(np.maximum.accumulate(x, axis=-1), y)
        assert np.all(np.diff(y, axis=-1) >= 0)
    # the first tile never changes; where the running max moves, codes match the tile-scaled ones
    same = (a.q_desc == b.q_desc)[0, 0]
    for t in np.nonzero(same)[0]:
        assert np.array_equal(a.q8[0, 0, 128 * t:128 * (t + 1)], b.q8[0, 0, 128 * t:128 * (t + 1)])
    assert same[0] and not same.all()


def test_prefix_scales_need_tiles():
    q, k, v = operands(7, 256)
    with pytest.raises(RuntimeError):
        oracle.prepare(q, k, v, prefix=True)
    with pytest.raises(RuntimeError):
        oracle.prepare(q, k, v, center=True, prefix=True)


def test_prefix_mean_is_the_first_tile_mean():
    """With prefix scales the mean key is the mean of the first 128 tokens:
    integer-valued keys make every partial sum exact and the mean of 128
    integers dyadic, so it is the exact rational rounded once; for N < 128 it
    is the mean of all N tokens."""
    g = np.random.default_rng(31)
    for N in (640, 100):
        k = g.integers(-1000, 1000, (1, 2, N, 64)).astype(np.float32)
        q = g.standard_normal((1, 4, N, 64)).astype(np.float32)
        p = oracle.prepare(q, k, k, center=True, tiles=True, prefix=True)
        n0 = min(N, 128)
        want = (k[:, :, :n0].astype(np.float64).sum(2) / n0).astype(np.float32)
        assert np.array_equal(p.k_mean, want)
        full = oracle.prepare(q, k, k, center=True)
        assert N <= 128 or not np.array_equal(full.k_mean, p.k_mean)


def test_prefix_mean_keeps_exact_attention():
    """The prefix mean is one vector subtracted from every key, so ideal
    attention on the centred keys equals ideal attention on the original keys
    (binary64, causal and not)."""
    q, k, v = operands(9, 384)
    p = oracle.prepare(q, k, v, center=True, tiles=True, prefix=True)
    kc = k.astype(np.float64) - p.k_mean[:, :, None, :].astype(np.float64)   # the shift, exact in binary64
    for causal in (True, False):
        np.testing.assert_allclose(oracle.attention_f64(q, kc, v, causal=causal),
                                   oracle.attention_f64(q, k, v, causal=causal), rtol=0, atol=1e-12)


def test_prefix_mean_and_scales_ignore_future_tiles():
    """Centred prefix prologue: changing tokens of tile 2 and later leaves the
    mean key and the codes and scales of tiles 0 and 1 untouched; with the
    full-sequence mean the same change moves the mean and every K code's
    centring."""
    N = 512
    q, k, v = operands(10, N)
    kw = dict(center=True, tiles=True, prefix=True, rotate=True, signs=signs(64))
    a = oracle.prepare(q, k, v, **kw)
    q2, k2 = q.copy(), k.copy()
    q2[:, :, 256:] *= np.float32(8.0)
    k2[:, :, 300:] += np.float32(5.0)
    b = oracle.prepare(q2, k2, v, **kw)
    assert np.array_equal(a.k_mean, b.k_mean)
    assert np.array_equal(a.q8[:, :, :256], b.q8[:, :, :256]) and np.array_equal(a.k8[:, :, :256], b.k8[:, :, :256])
    assert np.array_equal(a.q_desc[..., :2], b.q_desc[..., :2]) and np.array_equal(a.k_desc[..., :2], b.k_desc[..., :2])
    c = oracle.prepare(q, k, v, center=True, rotate=True, signs=signs(64))
    e = oracle.prepare(q2, k2, v, center=True, rotate=True, signs=signs(64))
    assert not np.array_equal(c.k_mean, e.k_mean)


@pytest.mark.parametrize("order", [0, 1])
def test_prefix_mean_output_close_to_ideal(order):
    """The centred prefix prologue followed by the tile-scaled loop stays
    within E4M3 noise of ideal attention on a shared-key workload."""
    w = synth.illustration(N=384, d=64, shared_norm=30.0)
    p = oracle.prepare(w.q, w.k, w.v, center=True, tiles=True, prefix=True, rotate=True, signs=w.signs)
    out = oracle.attention_fp8(p, kv_order=order, block_n=64).out
    ref = oracle.attention_f64(w.q, w.k, w.v, causal=True)
    assert oracle.head_errors(out, ref).max() < 0.1


def test_prefix_scales_ignore_future_tiles():
    """Changing tokens of tile 2 and later leaves the codes and scales of tiles
    0 and 1 untouched (the causality the prefix reading is for)."""
    N = 512
    q, k, v = operands(8, N)
    a = oracle.prepare(q, k, v, tiles=True, prefix=True)
    q2, k2 = q.copy(), k.copy()
    q2[:, :, 256:] *= np.float32(8.0)
    k2[:, :, 300:] += np.float32(5.0)
    b = oracle.prepare(q2, k2, v, tiles=True, prefix=True)
    assert np.array_equal(a.q8[:, :, :256], b.q8[:, :, :256]) and np.array_equal(a.k8[:, :, :256], b.k8[:, :, :256])
    assert np.array_equal(a.q_desc[..., :2], b.q_desc[..., :2]) and np.array_equal(a.k_desc[..., :2], b.k_desc[..., :2])
    assert not np.array_equal(a.q_desc[..., 2:], b.q_desc[..., 2:])
    # with full-sequence scales the same change reaches the early tiles' codes
    c, e = oracle.prepare(q, k, v), oracle.prepare(q2, k2, v)
    assert not np.array_equal(c.q8[:, :, :256], e.q8[:, :, :256])
