"""Stream semantics of the C-ABI: every entry point enqueues its kernels on the
stream it is given and nowhere else.  The prologue, the forward (timed and
dump forms) and the head error run back to back on a second stream, with no
host synchronisation between the calls, while unrelated work is queued on the
default stream; the results must equal the same calls on the default stream
bit for bit."""
import numpy as np
import pytest
import torch

import synth
from _gpu_helpers import dev, signs_dev

pytestmark = pytest.mark.gpu


def _run(pan, w, stream, d):
    B, hq, N, _ = w.q.shape
    hkv = w.k.shape[1]
    pipe = pan.AttnPipeline(B, hq, hkv, N, d)
    q, k, v = dev(w.q, "bf16"), dev(w.k, "bf16"), dev(w.v, "bf16")
    sg = signs_dev(w)
    ctx = torch.cuda.stream(stream) if stream is not None else torch.cuda.stream(torch.cuda.current_stream())
    with ctx:
        prep = pipe.prepare(q, k, v, rotate=True, center=True, signs=sg, stream=stream)
        kw = dict(p_scale=256.0, kv_order=1, block_n=128, causal=True, stream=stream)
        out = pipe.fwd(prep, **kw)
        rh = torch.zeros((B, hq, N), dtype=torch.int64, device="cuda")
        out_dump = pipe.fwd(prep, row_hash=rh, **kw)
        ref = torch.zeros((B, hq, N, d), dtype=torch.float64, device="cuda")
        rel = pipe.head_error(out, ref.copy_(out_dump), stream=stream)
    return [prep.q8, prep.k8, prep.v8t, prep.q_desc, prep.k_desc, prep.v_desc, out, out_dump, rh, rel]


@pytest.mark.parametrize("d", [64, 128])
def test_calls_on_a_second_stream_match_the_default_stream(d):
    import precision_attention_numerics_amd as pan
    w = synth.qwen_like(2, 6, 2, d, seed=950 + d, N=700, texts=2)
    print(f"[streams] d={d} shape={w.q.shape}", flush=True)
    want = _run(pan, w, None, d)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()      # default priority
    busy = torch.randn(4096, 4096, device="cuda")
    side.wait_stream(torch.cuda.current_stream())
    for _ in range(4):              # unrelated work on the default stream meanwhile
        busy = busy * 1.0001
    got = _run(pan, w, side, d)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for a, b in zip(want, got):
        assert a.shape == b.shape and a.dtype == b.dtype
        assert torch.equal(a.contiguous().view(torch.uint8), b.contiguous().view(torch.uint8))
    assert float(got[-1].abs().max()) == 0.0    # timed output against the dump form's: identical
