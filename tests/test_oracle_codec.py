"""Pins of the oracle's E4M3FN codec against the format's definition.

The format is fixed by the attention-numerics study page ("See the vectors and
the arithmetic": E4M3FN, round-to-nearest-even, saturation at +-448).  The
reference here is an independent nearest-value search over the finite values,
built directly from the format's value formula, not from the oracle."""
import os

import numpy as np
import pytest

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e4m3_facts.txt")


def finite_table():
    """(value, code) for the 127 non-negative finite E4M3FN codes, sorted by value."""
    vals, codes = [], []
    for code in range(0x7F):  # 0x7F is NaN
        e, m = code >> 3, code & 7
        vals.append(m * 2.0 ** -9 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7))
        codes.append(code)
    return np.array(vals), np.array(codes, np.uint8)


def nearest_search(x):
    """Brute-force reference: nearest finite value, ties to the even code,
    magnitudes above 448 saturate."""
    vals, codes = finite_table()
    a = np.abs(x.astype(np.float64))
    sign = np.where(np.signbit(x), 0x80, 0).astype(np.uint8)
    a = np.minimum(a, 448.0)
    hi = np.clip(np.searchsorted(vals, a, side="left"), 0, len(vals) - 1)
    lo = np.clip(hi - 1, 0, len(vals) - 1)
    dlo, dhi = a - vals[lo], vals[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & ((codes[hi] & 1) == 0))
    out = np.where(pick_hi, codes[hi], codes[lo])
    out = np.where(a == vals[hi], codes[hi], out)
    return (out | sign).astype(np.uint8)


def test_decode_all_codes(orc):
    vals, codes = finite_table()
    dec = orc.e4m3_decode(np.arange(256, dtype=np.uint8))
    assert np.array_equal(dec[:0x7F], vals.astype(np.float32))
    assert np.array_equal(dec[0x80:0xFF], -vals.astype(np.float32))
    assert np.isnan(dec[0x7F]) and np.isnan(dec[0xFF])


def _check_bits(orc, bits):
    for sgn in (0, 0x80000000):
        x = (bits | np.uint32(sgn)).view(np.float32)
        got = orc.e4m3_encode(x)
        ref = nearest_search(x)
        bad = np.nonzero(got != ref)[0]
        assert bad.size == 0, (sgn, x[bad[:5]], got[bad[:5]], ref[bad[:5]])


@pytest.mark.parametrize("e", [116, 117, 118, 121, 122, 127, 135, 136])
def test_encode_exhaustive_binade(orc, e):
    """Every binary32 of one binade, both signs: 2^-11, 2^-10 (the round-to-zero
    threshold), 2^-9 (smallest subnormal), the subnormal/normal boundary 2^-6
    and 2^-5, 1, [256, 512) (saturation starts above 448) and [512, 1024)."""
    _check_bits(orc, (np.uint32(e) << np.uint32(23)) | np.arange(1 << 23, dtype=np.uint32))


def test_encode_all_binades_edges(orc):
    """Every binade from 2^-27 to 2^15 at the mantissas where E4M3 rounding can
    change: each E4M3 step boundary and midpoint, plus or minus 3 ulps, and a
    stride through the rest."""
    low = np.arange(-3, 4, dtype=np.int64)
    anchors = np.arange(0, 1 << 23, 1 << 18, dtype=np.int64)     # boundaries and midpoints of 3-bit steps
    mant = np.unique(np.clip((anchors[:, None] + low[None, :]).ravel(), 0, (1 << 23) - 1))
    mant = np.unique(np.concatenate([mant, np.arange(0, 1 << 23, 997)])).astype(np.uint32)
    for e in range(100, 143):
        _check_bits(orc, (np.uint32(e) << np.uint32(23)) | mant)


def test_encode_random_full_range(orc):
    g = np.random.default_rng(5)
    x = g.integers(0, 2 ** 32, 2_000_000, dtype=np.uint64).astype(np.uint32).view(np.float32)
    x = x[~np.isnan(x)]
    assert np.array_equal(orc.e4m3_encode(x), nearest_search(x))


def test_golden_facts(orc):
    rows = []
    for line in open(GOLDEN):
        line = line.split("#")[0].strip()
        if not line:
            continue
        tok = line.split()
        rows.append((tok[0], int(tok[1], 16)))
    for s, code in rows:
        x = float.fromhex(s) if "0x" in s else float(s)
        assert int(orc.e4m3_encode(np.array([x], np.float32))[0]) == code, s


def test_roundtrip_codes(orc):
    c = np.array([c for c in range(256) if c & 0x7F != 0x7F], np.uint8)
    assert np.array_equal(orc.e4m3_encode(orc.e4m3_decode(c)), c)
