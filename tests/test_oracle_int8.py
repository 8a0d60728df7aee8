"""Pins of the oracle's INT8-QK mode (Q and K as int8 codes with a max-based
scale 127/A, V still E4M3; the INT8-QK / FP8-PV kernel family the
attention-numerics project page measures, whose quantisation the pages do not
give): round-to-nearest-even codes, reconstruction within half a step, and
every P~ code of a tiny head re-derived from exact integer scores."""
import numpy as np
import pytest

import oracle


def test_i8_codec_ties_to_even_and_clamps():
    x = np.array([0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 126.5, 127.5, 128.0, 200.0, -127.6, -1e30, 3.49999, 0.0])
    want = np.array([0, 2, 2, 0, -2, -2, 126, 127, 127, 127, -127, -127, 3, 0], np.int8)
    assert np.array_equal(oracle.i8_encode(x), want)


@pytest.mark.parametrize("tiles", [False, True])
def test_int8_codes_reconstruct_within_half_a_step(tiles):
    g = np.random.default_rng(11)
    q = g.standard_normal((1, 2, 300, 64)).astype(np.float32) * np.float32(3.0)
    k = g.standard_normal((1, 1, 300, 64)).astype(np.float32)
    v = g.standard_normal((1, 1, 300, 64)).astype(np.float32)
    p = oracle.prepare(q, k, v, tiles=tiles, int8=True)
    for x, codes, desc in ((q, p.q8, p.q_desc), (k, p.k8, p.k_desc)):
        c = codes.view(np.int8).astype(np.float64)
        dsc = np.repeat(desc, 128, axis=-1)[..., :300, None] if tiles else desc[..., None, None]
        err = np.abs(c * dsc - x)
        assert np.all(err <= dsc * 0.5 * (1 + 1e-5))
        assert np.abs(c).max() == 127
    # V keeps E4M3 codes with the 448 range
    assert np.abs(oracle.e4m3_decode(p.v8)).max() == 448.0


def test_int8_scores_are_exact_integer_dots():
    """A 3-token head (one block): every P~ code re-derived from the exact
    integer dot products of the int8 codes, c = (desc_q * desc_k) * RN32(scale
    * log2 e), x = fma(s, c, -RN32(m c)), p = RN32(2^x), P~ = E4M3(S p)."""
    g = np.random.default_rng(12)
    N, d, S = 3, 64, 256.0
    q = g.standard_normal((1, 1, N, d)).astype(np.float32)
    k = g.standard_normal((1, 1, N, d)).astype(np.float32)
    v = g.standard_normal((1, 1, N, d)).astype(np.float32)
    p = oracle.prepare(q, k, v, int8=True)
    r = oracle.attention_fp8(p, p_scale=S, causal=True, want_p=True)
    qi = p.q8[0, 0].view(np.int8).astype(np.int64)
    ki = p.k8[0, 0].view(np.int8).astype(np.int64)
    s = qi @ ki.T                                           # exact, |s| < 2^24
    ls2 = np.float32(float(np.float32(1 / np.sqrt(d))) * 1.4426950408889634)
    c = np.float32(np.float32(p.q_desc[0, 0] * p.k_desc[0, 0]) * ls2)
    for i in range(N):
        m = s[i, :i + 1].max()
        mc = np.float32(np.float64(m) * np.float64(c))
        x = (s[i, :i + 1].astype(np.float64) * np.float64(c) - np.float64(mc)).astype(np.float32)  # one rounding
        pj = oracle.exp2_rn32(x)
        codes = oracle.e4m3_encode(np.float32(S) * pj)
        assert np.array_equal(r.p[0, 0, i, :i + 1], codes), i
        assert not r.p[0, 0, i, i + 1:].any()


def test_int8_one_tile_is_the_per_head_path():
    g = np.random.default_rng(13)
    q, k, v = (g.standard_normal((1, 2, 100, 64)).astype(np.float32) for _ in range(3))
    k = k[:, :1]
    v = v[:, :1]
    a = oracle.prepare(q, k, v, int8=True)
    b = oracle.prepare(q, k, v, int8=True, tiles=True)
    assert np.array_equal(a.q8, b.q8) and np.array_equal(a.k8, b.k8)
    ra, rb = oracle.attention_fp8(a, want_p=True), oracle.attention_fp8(b, want_p=True)
    assert np.array_equal(ra.out, rb.out) and np.array_equal(ra.p, rb.p)
