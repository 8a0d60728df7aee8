"""fp8_attn_prepare_noalloc (the prologue on the library's static device
scratch) against fp8_attn_prepare with a caller workspace: bit-identical codes,
descales, mean key and status on two calls in a row, the second smaller, with
the first call's inputs eight times larger so that any scale maximum left over
in the shared scratch would show in the second call's descales.  The second
call adds no device memory."""
import numpy as np
import pytest
import torch

import synth
from _gpu_helpers import dev, signs_dev

pytestmark = pytest.mark.gpu


def _outputs(pipe, tiles):
    p = pipe.alloc_prepared(tiles=tiles)
    for t in (p.q8, p.k8, p.v8t, p.q_desc, p.k_desc, p.v_desc, p.k_mean):
        t.fill_(0x5A if t.dtype == torch.uint8 else float("nan"))
    return p


def _call(pan, w, dtype, flags, noalloc, prep):
    B, hq, N, d = w.q.shape
    hkv = w.k.shape[1]
    q, k, v = dev(w.q, dtype), dev(w.k, dtype), dev(w.v, dtype)
    shape = pan._abi.make_shape(B, hq, hkv, N, d, q, k, v)
    center = bool(flags & pan._abi.FP8A_CENTER_K)
    signs = signs_dev(w) if flags & pan._abi.FP8A_ROTATE_QK else None
    args = (shape, q, k, v, flags, signs, prep.q8, prep.k8, prep.v8t, prep.q_desc, prep.k_desc, prep.v_desc)
    if noalloc:
        pan._abi.fp8_attn_prepare_noalloc(*args, k_mean=prep.k_mean if center else None, status_word=prep.status)
    else:
        ws = torch.empty(max(pan._abi.prepare_workspace_bytes(shape, flags), 256), dtype=torch.uint8, device="cuda")
        pan._abi.fp8_attn_prepare(*args, k_mean=prep.k_mean if center else None, status_word=prep.status, workspace=ws)


def _same(a, b, center):
    for name in ("q8", "k8", "v8t", "q_desc", "k_desc", "v_desc", "status") + (("k_mean",) if center else ()):
        x, y = getattr(a, name).cpu().numpy(), getattr(b, name).cpu().numpy()
        assert np.array_equal(x.view(np.uint8), y.view(np.uint8)), f"{name} differs"


def test_noalloc_prepare_matches_the_workspace_entry_point_twice():
    import precision_attention_numerics_amd as pan
    A = pan._abi
    big = synth.long_context(seed=410, N=4096, hq=8, hkv=2, d=128)
    for x in (big.q, big.k, big.v):
        x *= 8.0                                   # exact in BF16
    small = synth.long_context(seed=411, N=1000, hq=4, hkv=1, d=64)
    cases = [(big, "bf16", A.FP8A_ROTATE_QK | A.FP8A_CENTER_K, False),
             (small, "f32", A.FP8A_ROTATE_QK | A.FP8A_CENTER_K | A.FP8A_TILE_SCALES, True)]
    for i, (w, dtype, flags, tiles) in enumerate(cases):
        B, hq, N, d = w.q.shape
        pipe = pan.AttnPipeline(B, hq, w.k.shape[1], N, d)
        shape = A.make_shape(B, hq, w.k.shape[1], N, d)
        assert A.prepare_workspace_bytes(shape, flags) <= A.NOALLOC_SCRATCH_BYTES
        want, got = _outputs(pipe, tiles), _outputs(pipe, tiles)
        _call(pan, w, dtype, flags, False, want)
        torch.cuda.synchronize()
        free0 = torch.cuda.mem_get_info()[0]
        _call(pan, w, dtype, flags, True, got)
        torch.cuda.synchronize()
        if i == 1:
            # the scratch is resident since the first call: nothing new on the device
            assert torch.cuda.mem_get_info()[0] == free0
        _same(got, want, center=True)
        print(f"[noalloc] call {i + 1}: B={B} hq={hq} N={N} d={d} {dtype} flags={flags} identical", flush=True)


def test_noalloc_prepare_rejects_a_shape_beyond_its_scratch():
    import precision_attention_numerics_amd as pan
    A = pan._abi
    shape = A.make_shape(1, 32, 8, 65536, 128)
    flags = A.FP8A_ROTATE_QK | A.FP8A_CENTER_K
    assert A.prepare_workspace_bytes(shape, flags) > A.NOALLOC_SCRATCH_BYTES
    t = torch.zeros(256, dtype=torch.uint8, device="cuda")
    with pytest.raises(A.Fp8AttnError) as e:
        A.fp8_attn_prepare_noalloc(shape, t.view(torch.bfloat16), t.view(torch.bfloat16), t.view(torch.bfloat16),
                                   flags, t.view(torch.int8), t, t, t, t.view(torch.float32), t.view(torch.float32),
                                   t.view(torch.float32))
    assert e.value.status == -5
