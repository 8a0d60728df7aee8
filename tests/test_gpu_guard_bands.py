"""Guard bands around every output buffer: each output of the prologue, the
forward (output, LSE, P~ dump, row checksums, underflow counts) and the head
error sits inside a larger allocation whose 4 KiB before and after hold a
sentinel byte; after the calls the sentinels must be intact.  Shapes are
ragged (N not a multiple of 128 or 64) and cover the pipelined kernel, the
dump / block-64 / head_dim-64 / per-tile / int8 forms and the binary32 P-cast
path, so a write past any buffer's end fails here."""
import numpy as np
import pytest
import torch

import synth
from _gpu_helpers import dev, signs_dev

pytestmark = pytest.mark.gpu
GUARD = 4096
SENTINEL = 0xA5


class Guarded:
    def __init__(self):
        self.bufs = []

    def __call__(self, shape, dtype):
        n = int(np.prod(shape)) * torch.empty((), dtype=dtype).element_size()
        raw = torch.full((GUARD + n + GUARD,), SENTINEL, dtype=torch.uint8, device="cuda")
        self.bufs.append((raw, n))
        return raw[GUARD:GUARD + n].view(dtype).view(shape)

    def check(self):
        torch.cuda.synchronize()
        for raw, n in self.bufs:
            lo, hi = raw[:GUARD], raw[GUARD + n:]
            assert bool((lo == SENTINEL).all()) and bool((hi == SENTINEL).all()), "guard band overwritten"


def _prepared(pan, g, B, hq, hkv, Np, d, tiles, int8):
    T = Np // 128 if tiles else 1
    return pan.Prepared(g((B, hq, Np, d), torch.uint8), g((B, hkv, Np, d), torch.uint8),
                        g((B, hkv, d, Np), torch.uint8), g((B * hq * T,), torch.float32),
                        g((B * hkv * T,), torch.float32), g((B * hkv,), torch.float32),
                        g((B * hkv * d,), torch.float32), g((1,), torch.int32), tiles, int8)


CASES = [  # (d, N, block_n, variant, dump)
    (128, 333, 128, "per_head", False),    # pipelined kernel
    (128, 333, 128, "per_head", True),     # dump variant
    (128, 200, 64, "per_head", False),     # block 64
    (64, 333, 128, "per_head", True),      # head_dim 64
    (128, 333, 128, "tiles", False),       # per-tile scales, pipelined
    (128, 333, 128, "int8", False),        # int8 scores
]


@pytest.mark.parametrize("d,N,bn,variant,dump", CASES)
def test_no_write_outside_the_outputs(d, N, bn, variant, dump):
    import precision_attention_numerics_amd as pan
    w = synth.qwen_like(1, 4, 2, d, seed=700 + d + N + bn, N=N, texts=1)
    B, hq, _, _ = w.q.shape
    hkv = w.k.shape[1]
    pipe = pan.AttnPipeline(B, hq, hkv, N, d)
    g = Guarded()
    tiles, int8 = variant == "tiles", variant == "int8"
    prep = _prepared(pan, g, B, hq, hkv, pipe.Np, d, tiles, int8)
    pipe.prepare(dev(w.q, "bf16"), dev(w.k, "bf16"), dev(w.v, "bf16"), rotate=True, center=True,
                 signs=signs_dev(w), prep=prep, tiles=tiles, int8=int8)
    out = g((B, hq, N, d), torch.float32)
    lse = g((B, hq, N), torch.float32)
    extra = {}
    if dump:
        extra = dict(p_dump=g((B, hq, N, N), torch.uint8), row_hash=g((B, hq, N), torch.int64),
                     row_zeros=g((B, hq, N), torch.int32), k_sink=4)
    pipe.fwd(prep, p_scale=256.0, kv_order=1, block_n=bn, causal=True, out=out, lse=lse, **extra)
    ref = torch.randn((B, hq, N, d), dtype=torch.float64, device="cuda")
    rel = g((B * hq,), torch.float64)
    pipe.head_error(out, ref, rel_err=rel)
    g.check()
    assert bool(torch.isfinite(out).all())


def test_pcast_path_writes_nothing_outside():
    import precision_attention_numerics_amd as pan
    N, d = 300, 64
    gen = np.random.default_rng(5)
    q, k, v = (torch.from_numpy(gen.standard_normal((1, 2, N, d)).astype(np.float32)).cuda() for _ in range(3))
    pipe = pan.AttnPipeline(1, 2, 2, N, d)
    g = Guarded()
    out, lse = g((1, 2, N, d), torch.float32), g((1, 2, N), torch.float32)
    pd, rh, rz = g((1, 2, N, N), torch.uint8), g((1, 2, N), torch.int64), g((1, 2, N), torch.int32)
    pipe.fwd_f32(q, k, v, p_scale=256.0, kv_order=1, block_n=128, causal=True, out=out, lse=lse, p_dump=pd,
                 row_hash=rh, row_zeros=rz, k_sink=4)
    g.check()
