"""Thin ctypes binding of libfp8attn.so (see include/fp8_attn.h).

Argument marshalling only: torch tensors are passed as device pointers plus
the current HIP stream; every step of the computation runs in the HIP
kernels.  The library must be built (``__graft_entry__.build()``); importing
this module without it raises, there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
import re

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# FP8A_LIB selects another build of the same sources (the host-sanitizer
# build, build.py --sanitize)
LIB_PATH = os.environ.get("FP8A_LIB") or os.path.join(_HERE, "libfp8attn.so")
HEADER = os.path.join(os.path.dirname(_HERE), "include", "fp8_attn.h")

FP8A_F32, FP8A_BF16, FP8A_F64, FP8A_E4M3, FP8A_I8QK = 0, 1, 2, 3, 4
FP8A_ROTATE_QK, FP8A_CENTER_K, FP8A_TILE_SCALES, FP8A_PREFIX_SCALES, FP8A_INT8_QK = 1, 2, 4, 8, 16
STATUS = {0: "FP8A_OK", -1: "FP8A_ERR_NULL", -2: "FP8A_ERR_SHAPE", -3: "FP8A_ERR_UNSUPPORTED",
          -4: "FP8A_ERR_PARAM", -5: "FP8A_ERR_WORKSPACE", -6: "FP8A_ERR_HIP"}


class Fp8AttnError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {STATUS.get(status, status)} ({strerror(status)})")


class Shape(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("hq", ctypes.c_int32), ("hkv", ctypes.c_int32),
                ("seqlen", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("q_stride", ctypes.c_int64 * 3), ("k_stride", ctypes.c_int64 * 3),
                ("v_stride", ctypes.c_int64 * 3)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                          "(hipcc --offload-arch=gfx950); there is no fallback path")
    lib = ctypes.CDLL(LIB_PATH)
    vp, sz, i32, i64, u32, f32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32, ctypes.c_float
    sp = ctypes.POINTER(Shape)
    lib.fp8_attn_padded_seqlen.argtypes = [i32]
    lib.fp8_attn_padded_seqlen.restype = i32
    lib.fp8_attn_prepare_workspace_bytes.argtypes = [sp, u32]
    lib.fp8_attn_prepare_workspace_bytes.restype = sz
    lib.fp8_attn_prepare.argtypes = [sp, ctypes.c_int, vp, vp, vp, u32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.fp8_attn_prepare.restype = ctypes.c_int
    lib.fp8_attn_prepare_noalloc.argtypes = [sp, ctypes.c_int, vp, vp, vp, u32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.fp8_attn_prepare_noalloc.restype = ctypes.c_int
    lib.fp8_attn_fwd.argtypes = [sp, ctypes.c_int, vp, vp, vp, vp, vp, vp, f32, f32, i32, i32, i32, vp, vp, vp, vp, vp,
                                 i32, vp]
    lib.fp8_attn_fwd.restype = ctypes.c_int
    lib.fp8_attn_fwd_tile_scaled.argtypes = [sp, vp, vp, vp, vp, vp, vp, f32, f32, i32, i32, i32, vp, vp, vp, vp,
                                             vp, i32, vp]
    lib.fp8_attn_fwd_tile_scaled.restype = ctypes.c_int
    lib.fp8_attn_head_error_workspace_bytes.argtypes = [sp, i64]
    lib.fp8_attn_head_error_workspace_bytes.restype = sz
    lib.fp8_attn_head_error.argtypes = [sp, vp, vp, ctypes.c_int, vp, i64, vp, vp, sz, vp]
    lib.fp8_attn_head_error.restype = ctypes.c_int
    lib.fp8_attn_strerror.argtypes = [ctypes.c_int]
    lib.fp8_attn_strerror.restype = ctypes.c_char_p
    lib.fp8_attn_build_info.argtypes = []
    lib.fp8_attn_build_info.restype = ctypes.c_char_p
    return lib


_lib = _load()


def header_functions() -> list[str]:
    """Names of the functions include/fp8_attn.h declares."""
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(fp8_attn_\w+)\s*\(", text)))


def strerror(status: int) -> str:
    return _lib.fp8_attn_strerror(int(status)).decode()


def build_info() -> str:
    """The loaded library's build identifier ("source_sha256=<hex> arch=gfx950")."""
    return _lib.fp8_attn_build_info().decode()


def _ptr(t: torch.Tensor | None):
    if t is None:
        return None
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def make_shape(batch, hq, hkv, seqlen, head_dim, q=None, k=None, v=None) -> Shape:
    s = Shape(batch, hq, hkv, seqlen, head_dim)
    for name, t in (("q_stride", q), ("k_stride", k), ("v_stride", v)):
        if t is not None:
            assert t.stride(-1) == 1, "channel axis must be contiguous"
            getattr(s, name)[:] = list(t.stride()[:3])
    return s


def padded_seqlen(n: int) -> int:
    return int(_lib.fp8_attn_padded_seqlen(int(n)))


def prepare_workspace_bytes(shape: Shape, flags: int) -> int:
    return int(_lib.fp8_attn_prepare_workspace_bytes(ctypes.byref(shape), int(flags)))


def head_error_workspace_bytes(shape: Shape, nrows: int) -> int:
    return int(_lib.fp8_attn_head_error_workspace_bytes(ctypes.byref(shape), int(nrows)))


def _dtype_code(t: torch.Tensor) -> int:
    return {torch.float32: FP8A_F32, torch.bfloat16: FP8A_BF16, torch.float64: FP8A_F64, torch.uint8: FP8A_E4M3}[t.dtype]


def fp8_attn_prepare(shape: Shape, q, k, v, flags: int, rot_signs, q8, k8, v8t, q_desc, k_desc, v_desc,
                     k_mean=None, status_word=None, workspace=None, stream=None) -> None:
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = _lib.fp8_attn_prepare(ctypes.byref(shape), _dtype_code(q), _ptr(q), _ptr(k), _ptr(v), int(flags),
                               _ptr(rot_signs), _ptr(q8), _ptr(k8), _ptr(v8t), _ptr(q_desc), _ptr(k_desc),
                               _ptr(v_desc), _ptr(k_mean), _ptr(status_word), _ptr(workspace), ws_bytes,
                               _stream(stream))
    if rc != 0:
        raise Fp8AttnError(rc, "fp8_attn_prepare")


def fp8_attn_prepare_noalloc(shape: Shape, q, k, v, flags: int, rot_signs, q8, k8, v8t, q_desc, k_desc, v_desc,
                             k_mean=None, status_word=None, stream=None) -> None:
    rc = _lib.fp8_attn_prepare_noalloc(ctypes.byref(shape), _dtype_code(q), _ptr(q), _ptr(k), _ptr(v), int(flags),
                                       _ptr(rot_signs), _ptr(q8), _ptr(k8), _ptr(v8t), _ptr(q_desc), _ptr(k_desc),
                                       _ptr(v_desc), _ptr(k_mean), _ptr(status_word), _stream(stream))
    if rc != 0:
        raise Fp8AttnError(rc, "fp8_attn_prepare_noalloc")


NOALLOC_SCRATCH_BYTES = 8 << 20


def fp8_attn_fwd(shape: Shape, qkv_dtype: int, q, k, v, q_desc, k_desc, v_desc, softmax_scale: float,
                 p_scale: float, kv_order: int, block_n: int, causal: int, out, lse=None, p_dump=None,
                 row_hash=None, row_zeros=None, k_sink: int = 0, stream=None) -> None:
    rc = _lib.fp8_attn_fwd(ctypes.byref(shape), int(qkv_dtype), _ptr(q), _ptr(k), _ptr(v), _ptr(q_desc),
                           _ptr(k_desc), _ptr(v_desc), float(softmax_scale), float(p_scale), int(kv_order),
                           int(block_n), int(causal), _ptr(out), _ptr(lse), _ptr(p_dump), _ptr(row_hash),
                           _ptr(row_zeros), int(k_sink), _stream(stream))
    if rc != 0:
        raise Fp8AttnError(rc, "fp8_attn_fwd")


def fp8_attn_fwd_tile_scaled(shape: Shape, q8, k8, v8t, q_desc, k_desc, v_desc, softmax_scale: float,
                             p_scale: float, kv_order: int, block_n: int, causal: int, out, lse=None, p_dump=None,
                             row_hash=None, row_zeros=None, k_sink: int = 0, stream=None) -> None:
    rc = _lib.fp8_attn_fwd_tile_scaled(ctypes.byref(shape), _ptr(q8), _ptr(k8), _ptr(v8t), _ptr(q_desc),
                                       _ptr(k_desc), _ptr(v_desc), float(softmax_scale), float(p_scale),
                                       int(kv_order), int(block_n), int(causal), _ptr(out), _ptr(lse),
                                       _ptr(p_dump), _ptr(row_hash), _ptr(row_zeros), int(k_sink), _stream(stream))
    if rc != 0:
        raise Fp8AttnError(rc, "fp8_attn_fwd_tile_scaled")


def fp8_attn_head_error(shape: Shape, out, ref, rows, nrows: int, rel_err, workspace, stream=None) -> None:
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = _lib.fp8_attn_head_error(ctypes.byref(shape), _ptr(out), _ptr(ref), _dtype_code(ref), _ptr(rows),
                                  int(nrows), _ptr(rel_err), _ptr(workspace), ws_bytes, _stream(stream))
    if rc != 0:
        raise Fp8AttnError(rc, "fp8_attn_head_error")
