"""CPU oracle for the causal FP8 (E4M3FN) attention forward.

TEST INFRASTRUCTURE ONLY.  Only the test suite, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py`` may import this package.  The HIP
library and its Python binding never import, link or call it, and it shares no
code with them.

What it computes (each function cites the passage it follows):

* :func:`attention_f64` -- ideal attention in binary64, the reference every
  head is measured against (attention-numerics project page, first section:
  each head's output is compared with exact causal attention in binary64).
* :func:`prepare` -- the quantisation prologue: per-(batch, head) max scales
  over the full sequence, optional mean-key centring before an optional
  random-sign Hadamard rotation of Q and K (never V), E4M3FN codes with
  round-to-nearest-even and saturation at +-448 (project page, second
  section; study page, "See the vectors and the arithmetic").
* :func:`attention_fp8` / :func:`attention_pcast_f32` -- the online softmax
  over KV blocks in forward or reverse order with P multiplied by the static
  scale S and cast to E4M3 before P.V, S divided out in the epilogue (P-Cast
  summary, Probleemstelling; Methodologie).
* :func:`head_errors`, :func:`harm_scores` -- the per-head metric: relative
  Frobenius output error per text, log(1 + e), mean over texts, rotated minus
  unrotated (study page, "What do these scores mean?").

Every function here is pinned by ``tests/test_oracle_*.py``
against closed forms, invariants, brute force or printed values.  The
matrix-unit score model of :func:`fp8_dot128` (``mode="mfma"``) is not
described by the pages (they fix only the E4M3 codec); it is pinned by cases
whose scores are derived by hand from each of its rules (pass order, group
truncation quantum, pass and running floors, per-pass rounding, sign of the
floor), and each plausible mistake in those rules is shown to fail one of them
(tests/test_oracle_score_model.py).  Parity unpinned against the pages: the
shared-key illustration's FP8 weights, whose vectors the page does not print.
"""
from __future__ import annotations

import ctypes
import functools
import os
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# FP8A_ORACLE_LIB selects another build of the same sources (the sanitizer
# build, oracle/build.py --sanitize)
_LIB_PATH = os.environ.get("FP8A_ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")
_lib = None

ROTATE = 1
CENTER = 2
TILE = 4
PREFIX = 8
INT8 = 16
TILE_TOKENS = 128
SCORE_MODES = {"mfma": 0, "exact": 1, "int8": 2}

_c_f32p = ctypes.POINTER(ctypes.c_float)
_c_f64p = ctypes.POINTER(ctypes.c_double)
_c_u8p = ctypes.POINTER(ctypes.c_uint8)
_c_i8p = ctypes.POINTER(ctypes.c_int8)
_c_i32p = ctypes.POINTER(ctypes.c_int32)
_c_u32p = ctypes.POINTER(ctypes.c_uint32)
_i64 = ctypes.c_int64


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _build
        _build.build()
    lib = ctypes.CDLL(_LIB_PATH)
    lib.orc_e4m3_encode_n.argtypes = [_c_f32p, _c_u8p, _i64]
    lib.orc_e4m3_decode_n.argtypes = [_c_u8p, _c_f32p, _i64]
    lib.orc_exp2_rn32_n.argtypes = [_c_f32p, _c_f32p, _i64]
    lib.orc_fp8_dot128.argtypes = [_c_u8p, _c_u8p, ctypes.c_int]
    lib.orc_fp8_dot128.restype = ctypes.c_float
    lib.orc_fwht_row.argtypes = [_c_f32p, _c_i8p, _i64]
    lib.orc_i8_encode.argtypes = [ctypes.c_float]
    lib.orc_i8_encode.restype = ctypes.c_int8
    lib.orc_attention_f64.argtypes = [_c_f64p, _c_f64p, _c_f64p, _i64, _i64, _i64, _i64, _i64,
                                      ctypes.c_int, ctypes.c_double, _c_i32p, _i64, _c_f64p, ctypes.c_int]
    lib.orc_prepare.argtypes = [_c_f32p, _c_f32p, _c_f32p, _i64, _i64, _i64, _i64, _i64, ctypes.c_uint32,
                                _c_i8p, _c_u8p, _c_u8p, _c_u8p, _c_f32p, _c_f32p, _c_f32p, _c_f32p]
    lib.orc_attention_fp8.argtypes = [_c_u8p, _c_u8p, _c_u8p, _c_f32p, _c_f32p, _c_f32p,
                                      _i64, _i64, _i64, _i64, _i64, ctypes.c_float, ctypes.c_float,
                                      ctypes.c_int, ctypes.c_int, ctypes.c_int, _c_i32p, _i64,
                                      _c_f32p, _c_u8p, _c_u32p, ctypes.c_int32, ctypes.c_int, ctypes.c_int, _c_f64p]
    lib.orc_attention_fp8_tiles.argtypes = lib.orc_attention_fp8.argtypes
    lib.orc_attention_fp8_rowhash.argtypes = [_c_u8p, _c_u8p, _c_u8p, _c_f32p, _c_f32p, _c_f32p,
                                              _i64, _i64, _i64, _i64, _i64, ctypes.c_float, ctypes.c_float,
                                              ctypes.c_int, ctypes.c_int, ctypes.c_int, _c_i32p, _i64,
                                              ctypes.POINTER(ctypes.c_uint64), _c_u32p, ctypes.c_int32,
                                              ctypes.c_int, ctypes.c_int]
    lib.orc_attention_pcast_f32.argtypes = [_c_f32p, _c_f32p, _c_f32p,
                                            _i64, _i64, _i64, _i64, _i64, ctypes.c_float, ctypes.c_float,
                                            ctypes.c_int, ctypes.c_int, ctypes.c_int, _c_i32p, _i64,
                                            _c_f32p, _c_u8p, _c_u32p, ctypes.c_int32, ctypes.c_int, ctypes.c_int,
                                            _c_f64p]
    _lib = lib
    return lib


def _p(a: np.ndarray | None, ctype):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctype)


def _threads(n: int | None) -> int:
    """Worker threads: ORACLE_THREADS if set, else the usable cores (at most 16)."""
    if n is not None:
        return int(n)
    env = os.environ.get("ORACLE_THREADS")
    if env:
        return int(env)
    return max(1, min(16, len(os.sched_getaffinity(0))))


def _check(rc: int, what: str):
    if rc != 0:
        raise RuntimeError(f"oracle {what} failed with code {rc}")


# ----------------------------------------------------------------- codec

def e4m3_encode(x) -> np.ndarray:
    """E4M3FN code of binary32 values: round to nearest even, saturate at +-448."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, np.uint8)
    _load().orc_e4m3_encode_n(_p(x.reshape(-1), _c_f32p), _p(out.reshape(-1), _c_u8p), x.size)
    return out


def i8_encode(x) -> np.ndarray:
    """int8 codes of binary32 values: round to nearest even, clamp to +-127."""
    x = np.asarray(x, dtype=np.float32)
    lib = _load()
    return np.array([lib.orc_i8_encode(float(v)) for v in x.ravel()], np.int8).reshape(x.shape)


def e4m3_decode(c) -> np.ndarray:
    """Value of E4M3FN codes as binary32 (0x7F/0xFF give NaN)."""
    c = np.ascontiguousarray(c, dtype=np.uint8)
    out = np.empty(c.shape, np.float32)
    _load().orc_e4m3_decode_n(_p(c.reshape(-1), _c_u8p), _p(out.reshape(-1), _c_f32p), c.size)
    return out


def exp2_rn32(x) -> np.ndarray:
    """2^x correctly rounded to binary32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, np.float32)
    _load().orc_exp2_rn32_n(_p(x.reshape(-1), _c_f32p), _p(out.reshape(-1), _c_f32p), x.size)
    return out


def fp8_dot128(a, b, mode: str = "mfma") -> np.float32:
    """Score of two E4M3 code vectors (length <= 128, zero-padded to 128)."""
    aa = np.zeros(128, np.uint8)
    bb = np.zeros(128, np.uint8)
    aa[:len(a)] = a
    bb[:len(b)] = b
    return np.float32(_load().orc_fp8_dot128(_p(aa, _c_u8p), _p(bb, _c_u8p), SCORE_MODES[mode]))


def fwht_rows(x, signs) -> np.ndarray:
    """Sign flip then unnormalised Sylvester Walsh-Hadamard transform of each
    row in binary32, stages h = 1, 2, ..., d/2."""
    x = np.array(x, dtype=np.float32, copy=True, order="C")
    s = np.ascontiguousarray(signs, dtype=np.int8)
    d = x.shape[-1]
    flat = x.reshape(-1, d)
    lib = _load()
    for r in range(flat.shape[0]):
        row = flat[r]
        lib.orc_fwht_row(row.ctypes.data_as(_c_f32p), _p(s, _c_i8p), d)
    return x


# ------------------------------------------------------------ attention

def _rows_arg(rows, N):
    if rows is None:
        return None, N
    r = np.ascontiguousarray(rows, dtype=np.int32)
    return r, r.size


def attention_f64(q, k, v, causal: bool = True, softmax_scale: float | None = None,
                  rows=None, nthreads: int | None = None) -> np.ndarray:
    """Ideal attention in binary64 on the original operands.

    q [B,Hq,N,d], k/v [B,Hkv,N,d] (any float dtype, widened exactly).
    Returns [B,Hq,nrows,d] float64."""
    q = np.ascontiguousarray(q, dtype=np.float64)
    k = np.ascontiguousarray(k, dtype=np.float64)
    v = np.ascontiguousarray(v, dtype=np.float64)
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    if softmax_scale is None:
        softmax_scale = 1.0 / np.sqrt(d)
    r, nrows = _rows_arg(rows, N)
    out = np.empty((B, Hq, nrows, d), np.float64)
    rc = _load().orc_attention_f64(_p(q, _c_f64p), _p(k, _c_f64p), _p(v, _c_f64p), B, Hq, Hkv, N, d,
                                   int(causal), float(softmax_scale), _p(r, _c_i32p), nrows,
                                   _p(out, _c_f64p), _threads(nthreads))
    _check(rc, "attention_f64")
    return out


@dataclass
class Prepared:
    q8: np.ndarray
    k8: np.ndarray
    v8: np.ndarray
    q_desc: np.ndarray
    k_desc: np.ndarray
    v_desc: np.ndarray
    k_mean: np.ndarray | None
    tiles: bool = False     # q_desc [B,Hq,T] / k_desc [B,Hkv,T] per 128-token tile
    int8: bool = False      # Q/K codes are int8 (scores: exact integer dot)


def prepare(q, k, v, rotate: bool = False, center: bool = False, signs=None, tiles: bool = False,
            prefix: bool = False, int8: bool = False) -> Prepared:
    """Quantisation prologue on binary32 operands (BF16 widened exactly).
    tiles: one Q/K scale per 128-token tile instead of per (batch, head) (the
    earlier emulator's granularity, attention-numerics project page, second
    section); V keeps per-head scales.  prefix (with tiles): tile t's Q/K scale
    from the largest maximum among tiles 0..t, so no scale depends on tokens
    past its tile; with center the mean key is taken over the first 128-token
    tile only (a shift common to every key that sees no later token).  int8: Q/K as int8 codes (scale 127/A,
    round to nearest even, clamp +-127), V still E4M3."""
    q = np.ascontiguousarray(q, dtype=np.float32)
    k = np.ascontiguousarray(k, dtype=np.float32)
    v = np.ascontiguousarray(v, dtype=np.float32)
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    s = None if signs is None else np.ascontiguousarray(signs, dtype=np.int8)
    q8 = np.empty(q.shape, np.uint8)
    k8 = np.empty(k.shape, np.uint8)
    v8 = np.empty(v.shape, np.uint8)
    T = (N + TILE_TOKENS - 1) // TILE_TOKENS if tiles else 1
    qd = np.empty(B * Hq * T, np.float32)
    kd = np.empty(B * Hkv * T, np.float32)
    vd = np.empty(B * Hkv, np.float32)
    km = np.empty(B * Hkv * d, np.float32) if center else None
    flags = ((ROTATE if rotate else 0) | (CENTER if center else 0) | (TILE if tiles else 0)
             | (PREFIX if prefix else 0) | (INT8 if int8 else 0))
    rc = _load().orc_prepare(_p(q, _c_f32p), _p(k, _c_f32p), _p(v, _c_f32p), B, Hq, Hkv, N, d, flags,
                             _p(s, _c_i8p), _p(q8, _c_u8p), _p(k8, _c_u8p), _p(v8, _c_u8p),
                             _p(qd, _c_f32p), _p(kd, _c_f32p), _p(vd, _c_f32p), _p(km, _c_f32p))
    _check(rc, "prepare")
    if tiles:
        return Prepared(q8, k8, v8, qd.reshape(B, Hq, T), kd.reshape(B, Hkv, T), vd.reshape(B, Hkv),
                        None if km is None else km.reshape(B, Hkv, d), True, int8)
    return Prepared(q8, k8, v8, qd.reshape(B, Hq), kd.reshape(B, Hkv), vd.reshape(B, Hkv),
                    None if km is None else km.reshape(B, Hkv, d), False, int8)


@dataclass
class LoopResult:
    out: np.ndarray
    p: np.ndarray | None
    row_zeros: np.ndarray | None
    lse: np.ndarray | None = None   # [B,Hq,nrows] binary64: (m*c + log2 l) * ln 2


def attention_fp8(prep: Prepared, softmax_scale: float | None = None, p_scale: float = 256.0,
                  kv_order: int = 0, block_n: int = 128, causal: bool = True, rows=None,
                  want_p: bool = False, k_sink: int = 0, score_mode: str = "mfma",
                  nthreads: int | None = None) -> LoopResult:
    """Online-softmax main loop on E4M3 codes.  kv_order 0 = forward, 1 = reverse.
    With per-tile descales (prep.tiles) the logit factor is formed per block
    and the running max kept in scaled units (orc_attention_fp8_tiles)."""
    B, Hq, N, d = prep.q8.shape
    Hkv = prep.k8.shape[1]
    if softmax_scale is None:
        softmax_scale = float(np.float32(1.0 / np.sqrt(d)))
    r, nrows = _rows_arg(rows, N)
    out = np.empty((B, Hq, nrows, d), np.float32)
    p = np.empty((B, Hq, nrows, N), np.uint8) if want_p else None
    z = np.empty((B, Hq, nrows), np.uint32)
    qd = np.ascontiguousarray(prep.q_desc, np.float32)
    kd = np.ascontiguousarray(prep.k_desc, np.float32)
    vd = np.ascontiguousarray(prep.v_desc, np.float32)
    fn = _load().orc_attention_fp8_tiles if prep.tiles else _load().orc_attention_fp8
    if prep.int8:
        score_mode = "int8"
    lse = np.empty((B, Hq, nrows), np.float64)
    rc = fn(_p(prep.q8, _c_u8p), _p(prep.k8, _c_u8p), _p(prep.v8, _c_u8p),
            _p(qd, _c_f32p), _p(kd, _c_f32p), _p(vd, _c_f32p),
            B, Hq, Hkv, N, d, float(softmax_scale), float(p_scale), int(kv_order),
            int(block_n), int(causal), _p(r, _c_i32p), nrows, _p(out, _c_f32p),
            _p(p, _c_u8p), _p(z, _c_u32p), int(k_sink), SCORE_MODES[score_mode],
            _threads(nthreads), _p(lse, _c_f64p))
    _check(rc, "attention_fp8")
    return LoopResult(out, p, z, lse)


def attention_fp8_rowhash(prep: Prepared, softmax_scale: float | None = None, p_scale: float = 256.0,
                          kv_order: int = 0, block_n: int = 128, causal: bool = True, rows=None,
                          k_sink: int = 0, score_mode: str = "mfma", nthreads: int | None = None):
    """The main loop's P~ codes only (per-head scales): per row the checksum
    row_hash(P~ row) and the count of zero codes among keys >= k_sink, without
    accumulating the output.  Returns (row_hash [B,Hq,nrows] uint64,
    row_zeros [B,Hq,nrows] uint32)."""
    if prep.tiles:
        raise ValueError("per-head scales only")
    B, Hq, N, d = prep.q8.shape
    Hkv = prep.k8.shape[1]
    if softmax_scale is None:
        softmax_scale = float(np.float32(1.0 / np.sqrt(d)))
    r, nrows = _rows_arg(rows, N)
    h = np.empty((B, Hq, nrows), np.uint64)
    z = np.empty((B, Hq, nrows), np.uint32)
    if prep.int8:
        score_mode = "int8"
    rc = _load().orc_attention_fp8_rowhash(
        _p(prep.q8, _c_u8p), _p(prep.k8, _c_u8p), _p(prep.v8, _c_u8p),
        _p(np.ascontiguousarray(prep.q_desc, np.float32), _c_f32p),
        _p(np.ascontiguousarray(prep.k_desc, np.float32), _c_f32p),
        _p(np.ascontiguousarray(prep.v_desc, np.float32), _c_f32p),
        B, Hq, Hkv, N, d, float(softmax_scale), float(p_scale), int(kv_order), int(block_n), int(causal),
        _p(r, _c_i32p), nrows, h.ctypes.data_as(ctypes.POINTER(ctypes.c_uint64)), _p(z, _c_u32p), int(k_sink),
        SCORE_MODES[score_mode], _threads(nthreads))
    _check(rc, "attention_fp8_rowhash")
    return h, z


def attention_pcast_f32(q, k, v, softmax_scale: float | None = None, p_scale: float = 256.0,
                        kv_order: int = 0, block_n: int = 128, causal: bool = False, rows=None,
                        want_p: bool = False, k_sink: int = 0, p_cast: bool = True,
                        nthreads: int | None = None) -> LoopResult:
    """Main loop with binary32 Q/K/V, only P cast (the P-Cast summary's
    simulation that follows the kernel step by step, Bijdragen item 4).  p_cast=False keeps P in binary32."""
    q = np.ascontiguousarray(q, dtype=np.float32)
    k = np.ascontiguousarray(k, dtype=np.float32)
    v = np.ascontiguousarray(v, dtype=np.float32)
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    if softmax_scale is None:
        softmax_scale = float(np.float32(1.0 / np.sqrt(d)))
    r, nrows = _rows_arg(rows, N)
    out = np.empty((B, Hq, nrows, d), np.float32)
    p = np.empty((B, Hq, nrows, N), np.uint8) if want_p else None
    z = np.empty((B, Hq, nrows), np.uint32)
    lse = np.empty((B, Hq, nrows), np.float64)
    rc = _load().orc_attention_pcast_f32(_p(q, _c_f32p), _p(k, _c_f32p), _p(v, _c_f32p),
                                         B, Hq, Hkv, N, d, float(softmax_scale), float(p_scale),
                                         int(kv_order), int(block_n), int(causal), _p(r, _c_i32p), nrows,
                                         _p(out, _c_f32p), _p(p, _c_u8p), _p(z, _c_u32p), int(k_sink),
                                         int(p_cast), _threads(nthreads), _p(lse, _c_f64p))
    _check(rc, "attention_pcast_f32")
    return LoopResult(out, p, z, lse)


# --------------------------------------------------------------- metrics

_M64 = (1 << 64) - 1


def splitmix64(seed: int, count: int) -> list[int]:
    """The first `count` outputs of the splitmix64 generator from `seed`
    (Steele, Lea and Flood, "Fast splittable pseudorandom number generators",
    OOPSLA 2014): add the golden-ratio increment to the state, then xor-shift
    and multiply twice."""
    out = []
    state = seed & _M64
    for _ in range(count):
        state = (state + 0x9E3779B97F4A7C15) & _M64
        z = state
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _M64
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _M64
        out.append(z ^ (z >> 31))
    return out


@functools.lru_cache(maxsize=8)
def key_weights(n: int) -> np.ndarray:
    """W_j = splitmix64 output j+1 from seed 0, made odd, for keys j < n
    (cached: do not modify the returned array)."""
    return np.array([w | 1 for w in splitmix64(0, n)], dtype=np.uint64)


def row_hash(p) -> np.ndarray:
    """Checksum of each row of P~ codes for verification (not part of the
    method): sum over keys j of code_j * W_j modulo 2^64.  p [..., N] uint8."""
    p = np.asarray(p)
    w = key_weights(p.shape[-1])
    with np.errstate(over="ignore"):
        return (p.astype(np.uint64) * w).sum(axis=-1, dtype=np.uint64)


def head_errors(o, ref) -> np.ndarray:
    """Relative Frobenius error per (batch, head): ||O - R||_F / ||R||_F over
    the head's [rows, d] block, in binary64."""
    o = np.asarray(o, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    num = np.sqrt(((o - r) ** 2).sum(axis=(-2, -1)))
    den = np.sqrt((r ** 2).sum(axis=(-2, -1)))
    return num / den


def mean_log1p(errs) -> np.ndarray:
    """log(1 + e) averaged over the text (batch) axis, per head."""
    return np.log1p(np.asarray(errs, dtype=np.float64)).mean(axis=0)


def harm_scores(err_rot, err_unrot) -> np.ndarray:
    """Rotated minus unrotated mean log1p error per head; > 0 means rotation
    harms the head (ties count as not harmed)."""
    return mean_log1p(err_rot) - mean_log1p(err_unrot)
