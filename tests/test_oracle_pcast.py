"""Pins of the P-cast main loop against the closed forms of the P-Cast
summary (gist.science, "P-Cast Precisie in FP8 Attention"), on the sink
generator of the P-collapse sweep (N = 4096, d = 128, 4-token sink block,
FP32 Q/K/V so only P is cast)."""
import math
import os

import numpy as np
import pytest
from scipy.stats import norm

import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pcast_closed_forms.txt")
LN_T = 10 * math.log(2)                  # 6.93: the 2^-10 round-to-zero threshold in natural-log units
ROWS = np.arange(0, 4096, 8)             # 512 query rows


def golden():
    out = {}
    for line in open(GOLDEN):
        if line.startswith("#") or "|" not in line:
            continue
        key, val, _ = [t.strip() for t in line.split("|", 2)]
        out[key] = val
    return out


def logits(w):
    q = w.q[0, 0].astype(np.float64)[ROWS]
    k = w.k[0, 0].astype(np.float64)
    return q @ k.T / np.sqrt(q.shape[-1])


@pytest.fixture(scope="module")
def sweep():
    return {delta: synth.pcast_sweep(float(delta)) for delta in (0, 4, 6, 7, 8, 10, 12)}


def test_golden_constants():
    g = golden()
    assert abs(float(g["ln_threshold"]) - LN_T) < 0.01
    assert g["round_to_zero_threshold"] == "2^-10"


def test_generator_logit_distribution(sweep):
    """Ordinary keys have N(0,1) logits given the query; sinks are raised by Delta."""
    z = logits(sweep[8])
    assert abs(z[:, 4:].mean()) < 0.01 and abs(z[:, 4:].std() - 1) < 0.01
    assert abs(z[:, :4].mean() - 8) < 0.1


@pytest.mark.parametrize("S,deltas", [(1.0, (4, 6, 7, 8)), (256.0, (10, 12)), (448.0, (10, 12))])
def test_forward_underflow_fraction_closed_form(orc, sweep, S, deltas):
    """Forward order: the fraction of non-sink P that casts to zero follows
    Phi(M - 6.93 - ln S) with M the running max set by the sink block
    (Theoretisch Kader, formula F(Delta, S) with M ~ Delta + delta_k)."""
    dk = float(golden()["delta_k_for_k4"])
    for delta in deltas:
        w = sweep[delta]
        r = orc.attention_pcast_f32(w.q, w.k, w.v, p_scale=S, kv_order=0, block_n=128, causal=False,
                                    rows=ROWS, k_sink=4)
        frac = r.row_zeros[0, 0].astype(np.float64) / (4096 - 4)
        z = logits(w)
        M = z[:, :128].max(axis=1)               # running max after the first (sink) block
        tight = norm.cdf(M - LN_T - math.log(S))
        assert abs(frac.mean() - tight.mean()) < 0.01, (S, delta, frac.mean(), tight.mean())
        printed = norm.cdf(delta + dk - 6.93 - math.log(S))
        # the printed form plugs in E[M]; the spread of the sink max (std ~0.7) makes
        # E[Phi(M - c)] differ from Phi(E[M] - c) by up to ~0.06 on the steep part
        assert abs(frac.mean() - printed) < 0.08, (S, delta, frac.mean(), printed)


def test_collapse_onset_near_delta_6_to_7_for_S1(orc, sweep):
    """At S = 1 the collapse switches on around Delta 6-7 (Theoretisch Kader)."""
    fr = {}
    for delta in (4, 6, 7, 8):
        w = sweep[delta]
        r = orc.attention_pcast_f32(w.q, w.k, w.v, p_scale=1.0, kv_order=0, causal=False, rows=ROWS, k_sink=4)
        fr[delta] = r.row_zeros.mean() / 4092
    assert fr[4] < 0.1 and fr[8] > 0.9 and 0.2 < fr[6] < 0.8


@pytest.mark.parametrize("delta", [0, 4, 8, 12])
def test_reverse_S256_no_underflow_outside_sink_block(orc, sweep, delta):
    """Reverse order with S = 256: no non-sink P outside the sink's KV block
    underflows (Optimalisatie 1, bound < 1e-12 per value)."""
    w = sweep[delta]
    r = orc.attention_pcast_f32(w.q, w.k, w.v, p_scale=256.0, kv_order=1, block_n=128, causal=False,
                                rows=ROWS, k_sink=128)
    assert int(r.row_zeros.sum()) == 0


@pytest.mark.parametrize("S", [1.0, 256.0])
def test_codes_monotone_in_delta_and_reverse_order_isolation(orc, sweep, S):
    """The sink generator draws the same numbers for every Delta and only adds
    Delta*sqrt(d)*u to the four sink keys, so every non-sink logit is the same
    at every Delta.  The running max that any block sees can only rise with
    Delta, so every non-sink P~ code is non-increasing in Delta, in both
    orders.  In reverse order the sinks' block (keys 0..127) is visited last,
    so every earlier block sees exactly the same running max at every Delta
    and its codes must not change at all."""
    ref = {}
    for delta in (0, 6, 12):
        w = sweep[delta]
        for order in (0, 1):
            r = orc.attention_pcast_f32(w.q, w.k, w.v, p_scale=S, kv_order=order, block_n=128, causal=False,
                                        rows=ROWS, want_p=True, k_sink=4)
            ref[(delta, order)] = r.p[0, 0].astype(np.int64)
    for order in (0, 1):
        for lo, hi in ((0, 6), (6, 12)):
            a, b = ref[(lo, order)][:, 4:], ref[(hi, order)][:, 4:]
            assert np.all(a & 0x80 == 0) and np.all(b & 0x80 == 0)     # probabilities: non-negative codes
            assert np.all(b <= a), (order, lo, hi, int((b > a).sum()))
    assert np.array_equal(ref[(0, 1)][:, 128:], ref[(12, 1)][:, 128:])
    # and the sinks' block does change (the test would be vacuous otherwise)
    assert not np.array_equal(ref[(0, 1)][:, 4:128], ref[(12, 1)][:, 4:128])
    assert not np.array_equal(ref[(0, 0)][:, 128:], ref[(12, 0)][:, 128:])


def test_dp_sawtooth(orc):
    """Normalised maximum quantisation step of P under scale S: 2^-4 for every
    power of two, 14% higher for S = 448 (Optimalisatie 2, item 2), measured by
    brute force over a dense grid of P in the normal range."""
    codes = np.arange(0x08, 0x7E, dtype=np.uint8)
    vals = orc.e4m3_decode(codes).astype(np.float64)
    steps = dict(zip(vals[:-1], np.diff(vals)))
    res = {}
    for S in (1.0, 2.0, 16.0, 128.0, 256.0, 448.0):
        worst = 0.0
        for j in range(-12, -1):
            p = np.linspace(2.0 ** j, 2.0 ** (j + 1), 4097)[:-1].astype(np.float32)
            y = (np.float32(S) * p).astype(np.float64)
            if y.min() < 2 ** -6 or y.max() >= 448:
                continue
            c = orc.e4m3_encode((np.float32(S) * p))
            lo = orc.e4m3_decode(np.where(orc.e4m3_decode(c) > y, c - 1, c).astype(np.uint8)).astype(np.float64)
            st = np.array([steps[v] for v in lo])
            worst = max(worst, (0.5 * st / (S * 2.0 ** j)).max())
        res[S] = worst
    for S in (1.0, 2.0, 16.0, 128.0, 256.0):
        assert res[S] == 2.0 ** -4
    assert abs(res[448.0] / 2.0 ** -4 - 8 / 7) < 1e-12
    assert abs(res[448.0] / 2.0 ** -4 - 1 - float(golden()["dp_448_excess"])) < 0.01


def test_normal_coverage_S256(orc):
    """With S = 256, every P >= 2^-14 casts to a normal code and the smallest
    non-zero P~/S is 2^-17 (Optimalisatie 2, item 3)."""
    p = np.geomspace(2.0 ** -14, 1.0, 200001).astype(np.float32)
    c = orc.e4m3_encode(np.float32(256.0) * p)
    assert np.all(((c >> 3) & 15) >= 1)
    assert orc.e4m3_encode(np.array([256 * 2.0 ** -18], np.float32))[0] == 0
    assert orc.e4m3_decode(orc.e4m3_encode(np.array([256 * 2.0 ** -17], np.float32)))[0] / 256 == 2.0 ** -17


def test_power_of_two_scale_exact(orc):
    """Multiplying P by S = 2^k and dividing again is exact in binary32; 448 is
    not (Optimalisatie 2, item 1)."""
    p = np.random.default_rng(0).random(1_000_000).astype(np.float32) + np.float32(1e-30)
    for S in (2.0, 256.0):
        assert np.array_equal((p * np.float32(S)) / np.float32(S), p)
    assert not np.array_equal(((p * np.float32(448)) / np.float32(448)), p)


def test_mse_claims_soft(orc, sweep):
    """Output MSE against exact attention at Delta = 7: forward S=1 is several
    times worse than forward S=256; forward S=448 is worse than S=256; reverse
    S=256 is close to forward S=256 (Experimentele Resultaten).  Asserted
    loosely; the values are printed."""
    w = sweep[7]
    ref = orc.attention_f64(w.q, w.k, w.v, causal=False, rows=ROWS)
    mse = {}
    for order, S in ((0, 1.0), (0, 256.0), (0, 448.0), (1, 256.0)):
        o = orc.attention_pcast_f32(w.q, w.k, w.v, p_scale=S, kv_order=order, causal=False, rows=ROWS).out
        mse[(order, S)] = float(((o - ref) ** 2).mean())
    print("MSE at Delta=7:", mse)
    assert mse[(0, 1.0)] / mse[(0, 256.0)] > 2.0
    assert mse[(0, 448.0)] > mse[(0, 256.0)]
    assert 0.5 < mse[(1, 256.0)] / mse[(0, 256.0)] < 2.0
