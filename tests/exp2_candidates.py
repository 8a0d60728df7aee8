"""The binary32 exponents x at which an exp2 that is off by a few units in
the last place could change an E4M3 code of S*2^x (helper of the fix-up
table tests; not collected by pytest).

For a P scale S the code of S*p is decided by the E4M3 rounding midpoints mu
(halfway between consecutive E4M3 values, and between 0 and the smallest
subnormal): p is on one side of mu/S or the other.  A p that is wrong by k
units in the last place can only flip a code when the correctly rounded p
lies within k units of such a boundary.  candidates(S) lists every x <= 0
whose correctly rounded 2^x (the oracle's exp2_rn32) lies within WINDOW
binary32 steps of a boundary: the complete set of inputs on which the
hardware exp2 has to be checked."""
from __future__ import annotations

import numpy as np

import oracle

WINDOW = 4


def e4m3_values() -> np.ndarray:
    """Every finite non-negative E4M3 value, ascending (codes 0x00..0x7E)."""
    return np.unique(oracle.e4m3_decode(np.arange(0x7F, dtype=np.uint8)).astype(np.float64))


def boundaries(S: float) -> np.ndarray:
    """Rounding midpoints of E4M3 below S, divided by S (binary64)."""
    v = e4m3_values()
    mid = 0.5 * (v[:-1] + v[1:])
    mid = mid[mid <= S]
    return mid / S


def _f32_steps(x: np.float32, lo: int, hi: int) -> np.ndarray:
    b = int(np.float32(x).view(np.uint32))
    return np.arange(b + lo, b + hi + 1, dtype=np.int64).astype(np.uint32).view(np.float32)


def candidates(S: float) -> np.ndarray:
    """Sorted unique binary32 x <= 0 with RN32(2^x) within WINDOW steps of a boundary."""
    out = []
    for b in boundaries(S):
        pb = np.float32(b)
        pw = _f32_steps(pb, -WINDOW - 1, WINDOW + 1)
        pw = pw[pw > 0]
        lo, hi = float(pw.min()), float(pw.max())
        # every x with RN32(2^x) in [lo, hi] lies in [log2(lo) - e, log2(hi) + e]
        # for e of a few binary32 steps of x; enumerate that range and filter
        x_lo, x_hi = np.float32(np.log2(lo)), np.float32(np.log2(hi))
        if x_lo > 0:
            continue
        # negative x: larger bit patterns are more negative
        b_hi = int(x_lo.view(np.uint32)) + 4 if x_lo < 0 else 4
        b_lo = int(x_hi.view(np.uint32)) - 4 if x_hi < 0 else 0
        if x_hi >= 0:
            b_lo = 0x80000000
        bits = np.arange(max(b_lo, 0x80000000), b_hi + 1, dtype=np.int64).astype(np.uint32)
        xs = bits.view(np.float32)
        p = oracle.exp2_rn32(xs)
        pl, ph = _f32_steps(pb, -WINDOW, WINDOW).min(), _f32_steps(pb, -WINDOW, WINDOW).max()
        keep = (p >= pl) & (p <= ph)
        out.append(xs[keep])
    if not out:
        return np.zeros(0, np.float32)
    xs = np.unique(np.concatenate(out))
    return xs[xs <= 0]


def p_codes(x: np.ndarray, S: float) -> np.ndarray:
    """E4M3 code of S * RN32(2^x) as the forward kernel forms it: the product
    is exact for a power-of-two S and rounded to binary32 once for S = 448."""
    p = oracle.exp2_rn32(x).astype(np.float32)
    return oracle.e4m3_encode((p * np.float32(S)).astype(np.float32))
