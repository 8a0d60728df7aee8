"""Seeded synthetic operands for the five workloads.

This module only draws inputs; it holds none of the attention method's
arithmetic.  Both the oracle side (tests) and the HIP side (tests, bench,
smoke) take their operands from here.  Everything is generated on the host
with numpy's Philox bit generator and returned as float32 arrays whose values
are exactly representable in the workload's storage type (BF16 workloads are
rounded to BF16 here, to nearest-even).

The pages measure real captures (private) from three public-domain books;
these generators stand in for them with the shapes and structure the pages
describe: a shared key component (attention-numerics study page, "A shared
key component should disappear"), outlier channels that motivate rotation
(project page, second section), RoPE'd BF16 operands from Qwen2.5-shaped
attention, and attention sinks with logit gap Delta (P-Cast summary,
Probleemstelling; Experimentele Resultaten).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

CONDITIONS = {
    "plain": dict(rotate=False, center=False),
    "rotated": dict(rotate=True, center=False),
    "centered": dict(rotate=False, center=True),
    "centered_rotated": dict(rotate=True, center=True),
}


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.Philox(seed))


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round binary32 values to the nearest BF16 value (ties to even); returns float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16 << 16
    return u.astype(np.uint32).view(np.float32).reshape(x.shape)


def rotation_signs(d: int, seed: int = 7) -> np.ndarray:
    """The fixed random sign vector of the Hadamard rotation (one per run)."""
    return np.where(rng(seed).random(d) < 0.5, -1, 1).astype(np.int8)


@dataclass
class Workload:
    name: str
    q: np.ndarray          # [B, Hq, N, d] float32 (exact in `dtype`)
    k: np.ndarray          # [B, Hkv, N, d]
    v: np.ndarray          # [B, Hkv, N, d]
    dtype: str             # "f32" or "bf16": storage type handed to the library
    causal: bool
    block_n: int
    p_scale: float
    kv_order: int          # 0 forward, 1 reverse
    conditions: tuple
    signs: np.ndarray
    meta: dict


def illustration(seed: int = 0, N: int = 256, d: int = 64, shared_norm: float = 20.0) -> Workload:
    """Single head, batch 1: Q, K, V ~ N(0,1); one shared vector of the given
    norm along the first coordinate added to every key."""
    g = rng(seed)
    q = g.standard_normal((1, 1, N, d), dtype=np.float32)
    k = g.standard_normal((1, 1, N, d), dtype=np.float32)
    v = g.standard_normal((1, 1, N, d), dtype=np.float32)
    k[..., 0] += np.float32(shared_norm)
    return Workload("illustration", q, k, v, "f32", True, 64, 256.0, 0, tuple(CONDITIONS), rotation_signs(d),
                    dict(seed=seed, N=N, d=d, shared_norm=shared_norm))


def _unit(g, n, d):
    x = g.standard_normal((n, d))
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def sink_heads(g, n_kv: int, group: int, N: int, d: int, delta: float, n_sink: int = 4):
    """Per KV head: a random unit direction u; queries q = u + sqrt(d-1) w with
    w a random unit vector orthogonal to u, so |q|^2 = d; keys ~ N(0, I) except
    the first n_sink keys, which get delta*sqrt(d)*u added.  Given q, the scaled
    logits q.k/sqrt(d) are N(0,1) for ordinary keys and delta + N(0,1) for the
    sinks."""
    q = np.empty((n_kv * group, N, d), np.float64)
    k = np.empty((n_kv, N, d), np.float64)
    for gh in range(n_kv):
        u = _unit(g, 1, d)[0]
        for j in range(group):
            w = g.standard_normal((N, d))
            w -= np.outer(w @ u, u)
            w /= np.linalg.norm(w, axis=-1, keepdims=True)
            q[gh * group + j] = u[None, :] + np.sqrt(d - 1.0) * w
        kk = g.standard_normal((N, d))
        kk[:n_sink] += delta * np.sqrt(d) * u[None, :]
        k[gh] = kk
    return q, k


def pcast_sweep(delta: float, seed: int = 100, N: int = 4096, d: int = 128) -> Workload:
    """P-collapse sweep point: one head, non-causal, FP32 operands; logits
    N(0,1) for ordinary keys and raised by delta for the 4-key sink block."""
    g = rng(seed)
    q, k = sink_heads(g, 1, 1, N, d, delta)
    v = g.standard_normal((1, 1, N, d))
    return Workload(f"pcast_sweep_delta{delta:g}", q[None].astype(np.float32), k[None].astype(np.float32),
                    v.astype(np.float32), "f32", False, 128, 256.0, 0, ("plain",), rotation_signs(d),
                    dict(seed=seed, N=N, d=d, delta=delta, n_sink=4))


def _rope(x: np.ndarray, base: float) -> np.ndarray:
    """Rotate-half RoPE over positions 0..N-1 (last two axes [N, d])."""
    N, d = x.shape[-2], x.shape[-1]
    half = d // 2
    inv = base ** (-np.arange(half, dtype=np.float64) / half)
    ang = np.arange(N, dtype=np.float64)[:, None] * inv[None, :]
    cos, sin = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * cos - x2 * sin, x2 * cos + x1 * sin], axis=-1)


def qwen_like(layers: int, hq: int, hkv: int, d: int, seed: int, N: int = 1024, texts: int = 3,
              name: str = "qwen", rope_base: float = 1.0e6) -> Workload:
    """Qwen2.5-shaped attention operands stacked as batch = layers * texts
    (layer-major).  Per (layer, text, head) Q, K, V ~ N(0,1); per (layer, KV
    head) 2-4 outlier channels scaled by U[10, 50] on K and on the group's
    query heads; RoPE; then a per-(layer, KV head) shared key vector of norm
    r * RMS|k| (r ~ U[5, 40] per layer) on the outlier channels, added to every
    key; BF16 rounding."""
    g = rng(seed)
    grp = hq // hkv
    B = layers * texts
    q = np.empty((B, hq, N, d), np.float32)
    k = np.empty((B, hkv, N, d), np.float32)
    v = np.empty((B, hkv, N, d), np.float32)
    meta_layers = []
    for L in range(layers):
        r_l = g.uniform(5.0, 40.0)
        outl = []
        for gh in range(hkv):
            n_o = int(g.integers(2, 5))
            ch = g.choice(d, n_o, replace=False)
            fac = g.uniform(10.0, 50.0, n_o)
            outl.append((ch, fac))
        shared = []
        for t in range(texts):
            b = L * texts + t
            qq = g.standard_normal((hq, N, d))
            kk = g.standard_normal((hkv, N, d))
            vv = g.standard_normal((hkv, N, d))
            for gh, (ch, fac) in enumerate(outl):
                kk[gh][:, ch] *= fac
                qq[gh * grp:(gh + 1) * grp][:, :, ch] *= fac
            qq = _rope(qq, rope_base)
            kk = _rope(kk, rope_base)
            if t == 0:
                shared = []
                for gh, (ch, fac) in enumerate(outl):
                    rms = np.sqrt((kk[gh] ** 2).sum(-1).mean())
                    u = np.zeros(d)
                    u[ch] = g.standard_normal(len(ch))
                    u *= r_l * rms / np.linalg.norm(u)
                    shared.append(u)
            for gh in range(hkv):
                kk[gh] += shared[gh][None, :]
            q[b] = round_bf16(qq.astype(np.float32))
            k[b] = round_bf16(kk.astype(np.float32))
            v[b] = round_bf16(vv.astype(np.float32))
        meta_layers.append(dict(r=float(r_l), outliers=[(c.tolist(), f.tolist()) for c, f in outl]))
    return Workload(name, q, k, v, "bf16", True, 128, 256.0, 1, tuple(CONDITIONS), rotation_signs(d),
                    dict(seed=seed, layers=layers, texts=texts, N=N, d=d, hq=hq, hkv=hkv, rope_base=rope_base,
                         layer_meta=meta_layers))


def qwen05b(seed: int = 200, layers: int = 24, N: int = 1024, texts: int = 3) -> Workload:
    """Qwen2.5-0.5B attention shape: 14 query heads, 2 KV heads, head_dim 64."""
    return qwen_like(layers, 14, 2, 64, seed, N=N, texts=texts, name="qwen2.5-0.5b")


def qwen15b(seed: int = 300, layers: int = 28, N: int = 1024, texts: int = 3) -> Workload:
    """Qwen2.5-1.5B attention shape: 12 query heads, 2 KV heads, head_dim 128."""
    return qwen_like(layers, 12, 2, 128, seed, N=N, texts=texts, name="qwen2.5-1.5b")


def long_context(seed: int = 400, N: int = 32768, hq: int = 32, hkv: int = 8, d: int = 128,
                 delta: float = 8.0) -> Workload:
    """Long-context throughput operands: batch 1, 32 query / 8 KV heads,
    head_dim 128, sink generator at delta with a 4-token sink block, V ~ N(0,1),
    rounded to BF16."""
    g = rng(seed)
    grp = hq // hkv
    q = np.empty((1, hq, N, d), np.float32)
    k = np.empty((1, hkv, N, d), np.float32)
    for gh in range(hkv):
        qq, kk = sink_heads(g, 1, grp, N, d, delta)
        q[0, gh * grp:(gh + 1) * grp] = round_bf16(qq.astype(np.float32))
        k[0, gh] = round_bf16(kk[0].astype(np.float32))
    v = round_bf16(g.standard_normal((1, hkv, N, d), dtype=np.float32))
    return Workload("long_context", q, k, v, "bf16", True, 128, 256.0, 1, ("rotated", "centered_rotated"),
                    rotation_signs(d), dict(seed=seed, N=N, hq=hq, hkv=hkv, d=d, delta=delta, n_sink=4))


def shared_key_vectors(seed: int, d: int = 8, keys: int = 4, grid: int = 8):
    """One query and `keys` keys of `d` channels for the study page's shared-key
    illustration ("01 / Synthetic illustration": four keys, eight channels).
    Entries are N(0,1) rounded to multiples of 2^-grid, so that adding an
    integer shared coordinate, averaging the keys and subtracting the mean
    are exact in binary32.  Returns (q [d], K [keys, d], signs [d]) as float32
    / int8; the shared first coordinate is added by the caller."""
    g = rng(seed)
    scale = float(2 ** grid)
    q = (np.round(g.standard_normal(d) * scale) / scale).astype(np.float32)
    K = (np.round(g.standard_normal((keys, d)) * scale) / scale).astype(np.float32)
    signs = np.where(g.random(d) < 0.5, -1, 1).astype(np.int8)
    return q, K, signs
