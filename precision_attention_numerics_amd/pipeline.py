"""Device-buffer plumbing around the C ABI: allocates with torch, then chains
fp8_attn_prepare -> fp8_attn_fwd -> fp8_attn_head_error on one stream."""
from __future__ import annotations

import math
from dataclasses import dataclass

import torch

from . import _abi


@dataclass
class Prepared:
    q8: torch.Tensor       # [B,hq,Np,d] uint8
    k8: torch.Tensor       # [B,hkv,Np,d] uint8
    v8t: torch.Tensor      # [B,hkv,d,Np] uint8
    q_desc: torch.Tensor   # [B*hq] float32, or [B*hq*T] with per-tile scales (T = Np/128)
    k_desc: torch.Tensor   # [B*hkv], or [B*hkv*T]
    v_desc: torch.Tensor   # [B*hkv]
    k_mean: torch.Tensor   # [B*hkv*d] (valid after a centred prepare)
    status: torch.Tensor   # [1] int32
    tiles: bool = False    # Q/K descales per 128-token tile
    int8: bool = False     # Q/K hold int8 codes (INT8-QK variant)


class AttnPipeline:
    def __init__(self, batch: int, hq: int, hkv: int, seqlen: int, head_dim: int, device="cuda"):
        self.B, self.hq, self.hkv, self.N, self.d = batch, hq, hkv, seqlen, head_dim
        self.device = torch.device(device)
        self.Np = _abi.padded_seqlen(seqlen)
        self.shape = _abi.make_shape(batch, hq, hkv, seqlen, head_dim)
        self._ws = {}

    def _workspace(self, key, nbytes: int) -> torch.Tensor:
        t = self._ws.get(key)
        if t is None or t.numel() < nbytes:
            t = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=self.device)
            self._ws[key] = t
        return t

    def alloc_prepared(self, tiles: bool = False, int8: bool = False) -> Prepared:
        B, hq, hkv, Np, d, dev = self.B, self.hq, self.hkv, self.Np, self.d, self.device
        T = Np // 128 if tiles else 1
        u8 = dict(dtype=torch.uint8, device=dev)
        f32 = dict(dtype=torch.float32, device=dev)
        return Prepared(torch.empty((B, hq, Np, d), **u8), torch.empty((B, hkv, Np, d), **u8),
                        torch.empty((B, hkv, d, Np), **u8), torch.empty(B * hq * T, **f32),
                        torch.empty(B * hkv * T, **f32), torch.empty(B * hkv, **f32),
                        torch.zeros(B * hkv * d, **f32), torch.zeros(1, dtype=torch.int32, device=dev), tiles, int8)

    def prepare(self, q, k, v, rotate: bool, center: bool, signs=None, prep: Prepared | None = None,
                stream=None, tiles: bool = False, prefix: bool = False, int8: bool = False) -> Prepared:
        """tiles: one Q/K scale per 128-token tile (FP8A_TILE_SCALES); the
        forward then uses fp8_attn_fwd_tile_scaled.  prefix (with tiles, not
        with center): tile t scaled by the largest maximum of tiles 0..t
        (FP8A_PREFIX_SCALES).  int8: Q/K as int8 codes (FP8A_INT8_QK); the
        forward then takes qkv_dtype FP8A_I8QK."""
        prep = prep or self.alloc_prepared(tiles, int8)
        if prep.tiles != tiles or prep.int8 != int8:
            raise ValueError("prepared buffers were allocated for another scale granularity or code type")
        flags = ((_abi.FP8A_ROTATE_QK if rotate else 0) | (_abi.FP8A_CENTER_K if center else 0)
                 | (_abi.FP8A_TILE_SCALES if tiles else 0) | (_abi.FP8A_PREFIX_SCALES if prefix else 0)
                 | (_abi.FP8A_INT8_QK if int8 else 0))
        shape = _abi.make_shape(self.B, self.hq, self.hkv, self.N, self.d, q, k, v)
        ws = self._workspace("prep", _abi.prepare_workspace_bytes(shape, flags))
        _abi.fp8_attn_prepare(shape, q, k, v, flags, signs if rotate else None, prep.q8, prep.k8, prep.v8t,
                              prep.q_desc, prep.k_desc, prep.v_desc, prep.k_mean if center else None,
                              prep.status, ws, stream)
        return prep

    def fwd(self, prep: Prepared, p_scale: float = 256.0, kv_order: int = 1, block_n: int = 128,
            causal: bool = True, softmax_scale: float | None = None, out=None, lse=None, p_dump=None,
            row_hash=None, row_zeros=None, k_sink: int = 0, stream=None) -> torch.Tensor:
        if softmax_scale is None:
            softmax_scale = 1.0 / math.sqrt(self.d)
        if out is None:
            out = torch.empty((self.B, self.hq, self.N, self.d), dtype=torch.float32, device=self.device)
        if prep.tiles:
            _abi.fp8_attn_fwd_tile_scaled(self.shape, prep.q8, prep.k8, prep.v8t, prep.q_desc, prep.k_desc,
                                          prep.v_desc, softmax_scale, p_scale, kv_order, block_n, int(causal),
                                          out, lse=lse, p_dump=p_dump, row_hash=row_hash, row_zeros=row_zeros,
                                          k_sink=k_sink, stream=stream)
        else:
            dtype = _abi.FP8A_I8QK if prep.int8 else _abi.FP8A_E4M3
            _abi.fp8_attn_fwd(self.shape, dtype, prep.q8, prep.k8, prep.v8t, prep.q_desc, prep.k_desc,
                              prep.v_desc, softmax_scale, p_scale, kv_order, block_n, int(causal), out, lse=lse,
                              p_dump=p_dump, row_hash=row_hash, row_zeros=row_zeros, k_sink=k_sink, stream=stream)
        return out

    def fwd_f32(self, q, k, v, p_scale: float = 256.0, kv_order: int = 0, block_n: int = 128,
                causal: bool = False, softmax_scale: float | None = None, out=None, lse=None, p_dump=None,
                row_hash=None, row_zeros=None, k_sink: int = 0, stream=None) -> torch.Tensor:
        if softmax_scale is None:
            softmax_scale = 1.0 / math.sqrt(self.d)
        if out is None:
            out = torch.empty((self.B, self.hq, self.N, self.d), dtype=torch.float32, device=self.device)
        _abi.fp8_attn_fwd(self.shape, _abi.FP8A_F32, q, k, v, None, None, None, softmax_scale, p_scale, kv_order,
                          block_n, int(causal), out, lse=lse, p_dump=p_dump, row_hash=row_hash, row_zeros=row_zeros,
                          k_sink=k_sink, stream=stream)
        return out

    def head_error(self, out, ref, rows=None, rel_err=None, stream=None) -> torch.Tensor:
        nrows = self.N if rows is None else int(rows.numel())
        ws = self._workspace("err", _abi.head_error_workspace_bytes(self.shape, nrows))
        if rel_err is None:
            rel_err = torch.empty(self.B * self.hq, dtype=torch.float64, device=self.device)
        _abi.fp8_attn_head_error(self.shape, out, ref, rows, nrows, rel_err, ws, stream)
        return rel_err
