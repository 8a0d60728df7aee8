"""The study page's synthetic illustration of a shared key component.

TEST INFRASTRUCTURE ONLY (part of the oracle; see oracle/__init__.py).

Attention-numerics study page, "01 / Synthetic illustration" and "See the
vectors and the arithmetic": one query and four keys of eight channels; the
keys share their first coordinate c, which shifts every score of the query by
the same amount, so exact softmax is unchanged by it.  Q and K each get one
maximum-based FP8 scale; an optional fixed random-sign Hadamard is applied to
both before rounding; E4M3FN with round-to-nearest-even and saturation at
+-448; dot products and softmax in binary64, scaling and conversion in
binary32.  Mean subtraction, when used, comes before the rotation.  The panel
stops at the attention weights (no rounding of probabilities or values, no
causal tiles).  Its error metric is the total variation between the FP8 and
the exact weights ("Weight error": the fraction of attention mass moved).

Readings where the page is silent: the softmax scale is 1/sqrt(8); the
Hadamard is the same unnormalised Sylvester transform as the main pipeline
with 1/sqrt(8) folded into the descale; the mean over the four keys is taken
in binary64 and rounded to binary32 before the subtraction in binary32.
"""
from __future__ import annotations

import numpy as np

from . import e4m3_decode, e4m3_encode, fwht_rows


def tv_distance(w, w_ref) -> float:
    """Total variation between two discrete distributions: half the L1 distance."""
    w = np.asarray(w, dtype=np.float64)
    w_ref = np.asarray(w_ref, dtype=np.float64)
    return 0.5 * float(np.abs(w - w_ref).sum())


def _softmax(z):
    z = np.asarray(z, dtype=np.float64)
    e = np.exp(z - z.max())
    return e / e.sum()


def exact_weights(q, K) -> np.ndarray:
    """Attention weights of the query over the keys in binary64."""
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    return _softmax(K @ q / np.sqrt(q.shape[-1]))


def _quantise(x, rotated: bool):
    """One max-based E4M3 scale for the whole array: values the codes stand for."""
    x = np.asarray(x, dtype=np.float32)
    A = np.float32(np.abs(x).max())
    if A == 0:
        inv, desc = np.float32(1), np.float32(1)
    else:
        inv = np.float32(np.float32(448.0) / A)
        desc = np.float32(A / np.float32(448.0))
    if rotated:
        desc = np.float32(desc * np.float32(1.0 / np.sqrt(x.shape[-1])))
    codes = e4m3_encode(x * inv)
    return e4m3_decode(codes).astype(np.float64) * np.float64(desc)


def fp8_weights(q, K, rotate: bool = False, center: bool = False, signs=None) -> np.ndarray:
    """Attention weights after the FP8 pipeline of the panel: optional mean-key
    subtraction, optional random-sign Hadamard of q and the keys, one E4M3
    scale for q and one for K, binary64 dot products and softmax."""
    q = np.asarray(q, dtype=np.float32)
    K = np.array(K, dtype=np.float32, copy=True)
    d = q.shape[-1]
    if center:
        mu = (K.astype(np.float64).sum(axis=0) / K.shape[0]).astype(np.float32)
        K = (K - mu).astype(np.float32)
    if rotate:
        q = fwht_rows(q[None, :], signs)[0]
        K = fwht_rows(K, signs)
    qd = _quantise(q, rotate)
    Kd = _quantise(K, rotate)
    return _softmax(Kd @ qd / np.sqrt(d))


def with_shared(K, c: float):
    """The keys with c added to their first coordinate."""
    K = np.array(K, dtype=np.float32, copy=True)
    K[:, 0] = K[:, 0] + np.float32(c)
    return K
