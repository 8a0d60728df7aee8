"""Pins of the oracle's RN32(2^x) against 50-digit decimal arithmetic."""
from decimal import Decimal, getcontext

import numpy as np

getcontext().prec = 60
LN2 = Decimal(2).ln()


def rn32_exact(x: float) -> np.float32:
    t = (Decimal(x) * LN2).exp()
    f = np.float32(float(t))
    # pick the nearest binary32 by exact comparison with the neighbours' midpoints
    cands = [np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))]
    best = min(cands, key=lambda c: (abs(Decimal(float(c)) - t), int(np.float32(c).view(np.uint32)) & 1))
    return np.float32(best)


def test_exp2_random(orc):
    g = np.random.default_rng(11)
    xs = np.concatenate([g.uniform(-30, 0.01, 1500), -g.exponential(0.3, 500)]).astype(np.float32)
    got = orc.exp2_rn32(xs)
    for x, y in zip(xs, got):
        assert y == rn32_exact(float(x)), x


def test_exp2_integers_exact(orc):
    xs = np.arange(-120, 10, dtype=np.float32)
    assert np.array_equal(orc.exp2_rn32(xs), np.ldexp(np.float32(1), xs.astype(np.int32)).astype(np.float32))


def test_exp2_near_e4m3_midpoints(orc):
    """x where 2^x lands within one binary32 ulp of an E4M3 rounding midpoint:
    the cases where a less accurate exp2 would flip a P code."""
    xs = []
    for mid in [0.96875, 0.71875, 0.5625 / 2, 0.0078125 * 1.0625, 0.90625, 0.59375]:
        x0 = np.float32(np.log2(mid))
        for k in range(-3, 4):
            xs.append(np.float32(x0 + np.float32(k) * np.spacing(x0)))
    xs += [np.float32(-0.0458037332), np.float32(-0.476438105), np.float32(-0.853158593), np.float32(-1.85315859)]
    xs = np.array(xs, np.float32)
    got = orc.exp2_rn32(xs)
    for x, y in zip(xs, got):
        assert y == rn32_exact(float(x)), x
