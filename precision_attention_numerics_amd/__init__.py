"""MI355X (gfx950) causal FP8 (E4M3FN) attention forward.

The computation lives in the HIP library libfp8attn.so behind the C ABI of
include/fp8_attn.h.  ``_abi`` is its thin ctypes binding (same names);
``pipeline`` allocates the device buffers with torch and chains the calls.
"""
from ._abi import (FP8A_BF16, FP8A_CENTER_K, FP8A_E4M3, FP8A_F32, FP8A_F64, FP8A_ROTATE_QK,  # noqa: F401
                   FP8A_I8QK, FP8A_INT8_QK, FP8A_PREFIX_SCALES, FP8A_TILE_SCALES, Fp8AttnError, Shape, fp8_attn_fwd, fp8_attn_fwd_tile_scaled,
                   fp8_attn_head_error, fp8_attn_prepare,
                   head_error_workspace_bytes, header_functions, make_shape, padded_seqlen,
                   prepare_workspace_bytes, strerror)
from .pipeline import AttnPipeline, Prepared  # noqa: F401
