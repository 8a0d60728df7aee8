"""Pins of the candidate set behind the exp2 fix-up table (tests/exp2_candidates.py):
the binary32 exponents on which a hardware exp2 must be checked against the
correctly rounded 2^x because an error of a few units in the last place of p
could change an E4M3 code of S*p.  The enumeration is compared with brute
force over every binary32 in two ranges, and the table's listed exponents are
shown to be such code-sensitive points."""
import numpy as np
import pytest

import oracle
import exp2_candidates as ec

P_SCALES = [float(2 ** k) for k in range(9)] + [448.0]
# exponents listed in the forward kernels' fix-up table (power-of-two S; S = 448)
LISTED = {"pow2": (0xBD3B9CB2, 0xBEF3EFB2), 448.0: (0xBF5A689A, 0xBFED344D)}


def _all_f32(lo: float, hi: float) -> np.ndarray:
    """Every binary32 in [lo, hi] for lo <= hi < 0."""
    a = int(np.float32(hi).view(np.uint32))
    b = int(np.float32(lo).view(np.uint32))
    return np.arange(a, b + 1, dtype=np.int64).astype(np.uint32).view(np.float32)


def _near_boundary(xs: np.ndarray, S: float) -> np.ndarray:
    p = oracle.exp2_rn32(xs).astype(np.float32)
    keep = np.zeros(xs.size, bool)
    for b in ec.boundaries(S):
        w = ec._f32_steps(np.float32(b), -ec.WINDOW, ec.WINDOW)
        keep |= (p >= w.min()) & (p <= w.max())
    return xs[keep]


@pytest.mark.parametrize("S", [256.0, 448.0, 1.0])
@pytest.mark.parametrize("lo,hi", [(-0.48, -0.47), (-0.06, -0.04), (-1.9, -1.8)])
def test_enumeration_matches_brute_force(S, lo, hi):
    xs = _all_f32(lo, hi)
    want = _near_boundary(xs, S)
    got = ec.candidates(S)
    got = got[(got >= np.float32(lo)) & (got <= np.float32(hi))]
    assert np.array_equal(np.sort(got), np.sort(want))


def test_boundaries_are_e4m3_midpoints():
    v = ec.e4m3_values()
    assert v[0] == 0 and v[1] == 2.0 ** -9 and v[-1] == 448.0 and v.size == 127
    b = ec.boundaries(256.0) * 256.0
    # each boundary encodes to the even neighbour (ties to even) and splits two codes
    for m in b[:40]:
        lo, hi = np.nextafter(np.float32(m), np.float32(0)), np.nextafter(np.float32(m), np.float32(1e9))
        assert oracle.e4m3_encode(np.float32(lo)) != oracle.e4m3_encode(np.float32(hi))


@pytest.mark.parametrize("S", P_SCALES)
def test_listed_exponents_are_code_sensitive(S):
    """Each listed x is a candidate, and moving 2^x by one binary32 step
    changes its code: a one-ulp exp2 error there is visible in P."""
    listed = LISTED[448.0] if S == 448.0 else LISTED["pow2"]
    cands = ec.candidates(S).view(np.uint32)
    for bits in listed:
        assert bits in cands
        x = np.array([bits], np.uint32).view(np.float32)
        p = oracle.exp2_rn32(x).astype(np.float32)
        c0 = ec.p_codes(x, S)[0]
        ups = oracle.e4m3_encode((np.nextafter(p, np.float32(2)) * np.float32(S)).astype(np.float32))[0]
        downs = oracle.e4m3_encode((np.nextafter(p, np.float32(0)) * np.float32(S)).astype(np.float32))[0]
        assert ups != c0 or downs != c0, hex(bits)


def test_candidate_counts_are_small():
    for S in P_SCALES:
        n = ec.candidates(S).size
        assert 500 < n < 2000, (S, n)
