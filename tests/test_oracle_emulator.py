"""Pins of the oracle's quantised-pipeline emulator (prologue and main loop).

References: invariants the pages state (V never rotated, centring touches K
only, one max-based scale per head), closed-form error bounds of E4M3, and
reduction to plain binary32/binary64 attention when the cast is removed."""
import numpy as np
import pytest

import synth


def rand32(shape, seed, scale=1.0):
    return (np.random.default_rng(seed).standard_normal(shape) * scale).astype(np.float32)


def dequant(codes, desc, orc):
    return orc.e4m3_decode(codes).astype(np.float64) * desc[..., None, None]


# ------------------------------------------------------------------ prologue

def test_mean_key_exact_on_integers(orc):
    """Integer-valued keys: every partial sum is exact, so the mean is the
    exact rational rounded once (N = 256: the mean is dyadic and representable)."""
    g = np.random.default_rng(1)
    k = g.integers(-1000, 1000, (1, 2, 256, 16)).astype(np.float32)
    prep = orc.prepare(k[:, :1].repeat(2, 1), k, k, center=True)
    assert np.array_equal(prep.k_mean, (k.astype(np.float64).sum(2) / 256).astype(np.float32))


def test_mean_key_ragged_within_half_ulp(orc):
    k = rand32((1, 1, 197, 32), 2, 3.0) + np.float32(40.0)
    prep = orc.prepare(k, k, k, center=True)
    exact = np.array([np.sum(k[0, 0, :, c].astype(np.float64)) for c in range(32)]) / 197
    err = np.abs(prep.k_mean[0, 0].astype(np.float64) - exact)
    assert np.all(err <= 0.5 * np.spacing(np.abs(prep.k_mean[0, 0])) * (1 + 1e-6))


@pytest.mark.parametrize("cond", list(synth.CONDITIONS))
def test_amax_element_saturates_to_448_and_bounds(orc, cond):
    """One maximum-based scale per (batch, head): the largest transformed
    magnitude maps to +-448 (0x7E/0xFE); every other element is within E4M3's
    relative half-step 2^-4 (normal range) or half the subnormal quantum."""
    w = synth.illustration(N=100, d=64)
    flags = synth.CONDITIONS[cond]
    prep = orc.prepare(w.q, w.k, w.v, signs=w.signs, **flags)
    for codes in (prep.q8, prep.k8, prep.v8):
        per_head = codes.reshape(codes.shape[0] * codes.shape[1], -1) & 0x7F
        assert np.all(per_head.max(axis=1) == 0x7E)
    d = w.q.shape[-1]
    # dequantised Q against the transformed Q (rotation folded 1/sqrt(d) into the descale)
    x = w.q.astype(np.float64)
    if flags["rotate"]:
        x = orc.fwht_rows(w.q, w.signs).astype(np.float64) / np.sqrt(d)
    deq = dequant(prep.q8, prep.q_desc, orc)
    desc_unit = prep.q_desc[..., None, None] / (1 / np.sqrt(d) if flags["rotate"] else 1.0)
    bound = np.maximum(2.0 ** -4 * np.abs(x), 2.0 ** -10 * desc_unit / (np.sqrt(d) if flags["rotate"] else 1.0))
    assert np.all(np.abs(deq - x) <= bound * 1.0001 + 1e-7 * np.abs(x))


def test_v_never_rotated_and_centering_touches_k_only(orc):
    w = synth.illustration(N=128, d=64)
    plain = orc.prepare(w.q, w.k, w.v, signs=w.signs)
    rot = orc.prepare(w.q, w.k, w.v, signs=w.signs, rotate=True)
    cen = orc.prepare(w.q, w.k, w.v, signs=w.signs, center=True)
    assert np.array_equal(plain.v8, rot.v8) and np.array_equal(plain.v_desc, rot.v_desc)
    assert np.array_equal(plain.q8, cen.q8) and np.array_equal(plain.v8, cen.v8)
    assert not np.array_equal(plain.k8, cen.k8)


def test_descale_formula(orc):
    w = synth.illustration(N=64, d=64)
    for rotate in (False, True):
        prep = orc.prepare(w.q, w.k, w.v, signs=w.signs, rotate=rotate)
        xq = orc.fwht_rows(w.q, w.signs) if rotate else w.q
        A = np.float32(np.abs(xq).max())
        desc = np.float32(A / np.float32(448.0))
        if rotate:
            desc = np.float32(desc * np.float32(1 / np.sqrt(64.0)))
        assert prep.q_desc[0, 0] == desc


def test_zero_head_gets_unit_scale(orc):
    q = np.zeros((1, 1, 8, 64), np.float32)
    prep = orc.prepare(q, q, q)
    assert prep.q_desc[0, 0] == 1.0 and np.all(prep.q8 == 0)


def test_centering_then_rotation_restores_shared_key_case(orc):
    """With a large shared key component, centring makes the dequantised scores
    match exact scores far better than without (the pages' mechanism)."""
    w = synth.illustration(N=256, d=64, shared_norm=40.0)
    exact = w.q[0, 0].astype(np.float64) @ w.k[0, 0].astype(np.float64).T
    exact -= exact.mean(axis=1, keepdims=True)
    errs = {}
    for name, fl in synth.CONDITIONS.items():
        p = orc.prepare(w.q, w.k, w.v, signs=w.signs, **fl)
        sq = orc.e4m3_decode(p.q8[0, 0]).astype(np.float64)
        sk = orc.e4m3_decode(p.k8[0, 0]).astype(np.float64)
        s = (sq @ sk.T) * p.q_desc[0, 0] * p.k_desc[0, 0]
        s -= s.mean(axis=1, keepdims=True)
        errs[name] = np.abs(s - exact).mean()
    assert errs["centered"] < errs["plain"] and errs["centered_rotated"] < errs["rotated"]


# ----------------------------------------------------------------- main loop

@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("order", [0, 1])
@pytest.mark.parametrize("bn", [16, 64, 1000])
def test_identity_cast_equals_plain_attention(orc, causal, order, bn):
    """Without the E4M3 cast the online softmax is plain binary32 softmax(QK^T)V:
    it matches binary64 attention to binary32 rounding, for either visiting
    order and any block size (textbook online-softmax identity)."""
    q, k, v = rand32((1, 2, 150, 32), 3), rand32((1, 1, 150, 32), 4), rand32((1, 1, 150, 32), 5)
    ref = orc.attention_f64(q, k, v, causal=causal)
    got = orc.attention_pcast_f32(q, k, v, causal=causal, kv_order=order, block_n=bn, p_cast=False).out
    np.testing.assert_allclose(got, ref, rtol=2e-5, atol=2e-6)


def test_rows_subset_and_masked_codes(orc):
    w = synth.illustration(N=200, d=64)
    prep = orc.prepare(w.q, w.k, w.v, signs=w.signs, rotate=True)
    full = orc.attention_fp8(prep, p_scale=256.0, kv_order=0, block_n=64, causal=True, want_p=True)
    rows = np.array([5, 199, 63, 64, 0])
    sub = orc.attention_fp8(prep, p_scale=256.0, kv_order=0, block_n=64, causal=True, rows=rows, want_p=True)
    assert np.array_equal(sub.out, full.out[:, :, rows]) and np.array_equal(sub.p, full.p[:, :, rows])
    P = full.p[0, 0]
    assert np.all(np.triu(P, 1) == 0)                       # masked keys dumped as 0
    assert np.all((P == 0x78).any(axis=1))                  # the row max always casts to S = 256


def test_fp8_output_close_to_ideal(orc):
    w = synth.illustration(N=256, d=64)
    ref = orc.attention_f64(w.q, w.k, w.v, causal=True)
    for name, fl in synth.CONDITIONS.items():
        prep = orc.prepare(w.q, w.k, w.v, signs=w.signs, **fl)
        o = orc.attention_fp8(prep, p_scale=256.0, kv_order=0, block_n=64, causal=True).out
        e = orc.head_errors(o, ref)
        assert np.all(e < 0.15), (name, e)


def test_head_error_metric(orc):
    r = np.random.default_rng(0).standard_normal((2, 3, 10, 4))
    eps = np.array([[0.1, 0.02, 0.0], [0.5, 1e-3, 0.25]])
    o = r * (1 + eps[..., None, None])
    np.testing.assert_allclose(orc.head_errors(o, r), np.abs(eps), rtol=1e-12, atol=1e-15)
    hs = orc.harm_scores(np.array([[0.2], [0.1]]), np.array([[0.1], [0.1]]))
    np.testing.assert_allclose(hs, [(np.log1p(0.2) + np.log1p(0.1)) / 2 - np.log1p(0.1)])


# --------------------------------------------------------------- score model

def test_score_exact_mode_matches_fractions(orc):
    from fractions import Fraction
    g = np.random.default_rng(9)
    vals = orc.e4m3_decode(np.arange(256, dtype=np.uint8))
    for _ in range(200):
        a = g.integers(0, 256, 128).astype(np.uint8)
        b = g.integers(0, 256, 128).astype(np.uint8)
        a[(a & 0x7F) == 0x7F] = 0
        b[(b & 0x7F) == 0x7F] = 0
        s = sum(Fraction(float(vals[x])) * Fraction(float(vals[y])) for x, y in zip(a, b))
        assert orc.fp8_dot128(a, b, "exact") == np.float32(float(s)) or abs(float(s)) > 2 ** 24


def test_score_matrix_model_reduces_to_exact_without_truncation(orc):
    """When every group of eight products spans fewer than 13 binades and all
    partial sums fit in 24 bits, the matrix-unit precision equals the exact
    rounded dot product."""
    g = np.random.default_rng(10)
    for _ in range(300):
        a = (g.integers(0, 2, 128) << 7 | (0x38 + g.integers(0, 8, 128))).astype(np.uint8)   # [1, 2)
        b = (g.integers(0, 2, 128) << 7 | (0x38 + g.integers(0, 16, 128))).astype(np.uint8)  # [1, 4)
        assert orc.fp8_dot128(a, b, "mfma") == orc.fp8_dot128(a, b, "exact")


def test_score_matrix_model_symmetries(orc):
    g = np.random.default_rng(12)
    for _ in range(300):
        a = g.integers(0, 256, 128).astype(np.uint8)
        b = g.integers(0, 256, 128).astype(np.uint8)
        a[(a & 0x7F) == 0x7F] = 0
        b[(b & 0x7F) == 0x7F] = 0
        s = orc.fp8_dot128(a, b)
        assert orc.fp8_dot128(b, a) == s
        ex = float(orc.fp8_dot128(a, b, "exact"))
        vals = np.abs(orc.e4m3_decode(a).astype(np.float64) * orc.e4m3_decode(b))
        bound = sum(8 * vals[16 * i: 16 * i + 16].max() * 2.0 ** -12 for i in range(8)) + 16 * np.spacing(np.float32(abs(ex) + vals.sum()))
        assert abs(float(s) - ex) <= bound


@pytest.mark.parametrize("order", [0, 1])
def test_lse_is_the_logsumexp_of_the_loop_logits(orc, order):
    """The loop's LSE, (running max in base-2 units + log2 l) * ln 2, equals
    the binary64 log-sum-exp of its own scaled logits s*c*ln 2 (scores from
    the matrix-unit model) to binary32 rounding of l; and with binary32
    operands and no cast, the log-sum-exp of the plain logits q.k/sqrt(d)."""
    w = synth.illustration(N=96, d=64)
    prep = orc.prepare(w.q, w.k, w.v, signs=w.signs, rotate=True)
    res = orc.attention_fp8(prep, kv_order=order, block_n=64, causal=True)
    ls2 = np.float32(np.float64(np.float32(1 / np.sqrt(64))) * 1.4426950408889634)
    c = np.float64(np.float32(np.float32(prep.q_desc[0, 0]) * np.float32(prep.k_desc[0, 0])) * ls2)
    for i in (0, 1, 37, 95):
        s = np.array([float(orc.fp8_dot128(prep.q8[0, 0, i], prep.k8[0, 0, j])) for j in range(i + 1)])
        z = s * c * np.log(2.0)
        want = np.log(np.exp(z - z.max()).sum()) + z.max()
        assert abs(res.lse[0, 0, i] - want) <= 1e-6 * max(1.0, abs(want)), (i, res.lse[0, 0, i], want)
    q, k, v = rand32((1, 1, 80, 32), 3), rand32((1, 1, 80, 32), 4), rand32((1, 1, 80, 32), 5)
    r = orc.attention_pcast_f32(q, k, v, causal=True, kv_order=order, block_n=16, p_cast=False)
    z = (q[0, 0].astype(np.float64) @ k[0, 0].astype(np.float64).T) / np.sqrt(32)
    z = np.where(np.tril(np.ones((80, 80), bool)), z, -np.inf)
    want = np.log(np.exp(z - z.max(1, keepdims=True)).sum(1)) + z.max(1)
    np.testing.assert_allclose(r.lse[0, 0], want, rtol=2e-6, atol=2e-6)
