"""GPU parity of the INT8-QK variant (Q/K as int8 codes with a max-based
scale 127/A per (batch, head), exact integer scores on the int8 matrix cores;
P~ and V in E4M3 as in the FP8 path): prologue codes and descales bit-exact,
every P~ code, underflow count and row checksum equal to the oracle's, outputs
within 2e-3 per head, and the dump variant equal to the timed one."""
import numpy as np
import pytest
import torch

import oracle
import synth
from _gpu_helpers import compare_prepared, dev, max_head_rel, p_mismatch, signs_dev

pytestmark = pytest.mark.gpu
TOL_O = 2e-3


@pytest.fixture(scope="module")
def pan():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    import precision_attention_numerics_amd as pan
    return pan


def run_int8(pan, w, cond, p_scale=256.0, kv_order=1, block_n=128, causal=True, rows=None, k_sink=4):
    flags = synth.CONDITIONS[cond]
    B, hq, N, d = w.q.shape
    hkv = w.k.shape[1]
    pipe = pan.AttnPipeline(B, hq, hkv, N, d)
    print(f"int8 {w.name} {cond} S={p_scale} order={kv_order} bc={block_n} causal={causal} shape={w.q.shape}",
          flush=True)
    gp = pipe.prepare(dev(w.q, w.dtype), dev(w.k, w.dtype), dev(w.v, w.dtype), signs=signs_dev(w), int8=True,
                      **flags)
    op = oracle.prepare(w.q, w.k, w.v, signs=w.signs, int8=True, **flags)
    torch.cuda.synchronize()
    compare_prepared(gp, op, N, flags["center"])
    kw = dict(p_scale=p_scale, kv_order=kv_order, block_n=block_n, causal=causal)
    pd = torch.zeros((B, hq, N, N), dtype=torch.uint8, device="cuda") if rows is None else None
    rz = torch.zeros((B, hq, N), dtype=torch.int32, device="cuda")
    rh = torch.zeros((B, hq, N), dtype=torch.int64, device="cuda")
    out = pipe.fwd(gp, p_dump=pd, row_hash=rh, row_zeros=rz, k_sink=k_sink, **kw)
    out_nodump = pipe.fwd(gp, **kw)
    torch.cuda.synchronize()
    ref = oracle.attention_fp8(op, rows=rows, want_p=True, k_sink=k_sink, **kw)
    o = out.cpu().numpy()
    assert np.array_equal(o, out_nodump.cpu().numpy()), "dump and timed variants differ"
    Z = rz.cpu().numpy().astype(np.uint32)
    H = rh.cpu().numpy().view(np.uint64)
    if rows is not None:
        o, Z, H = o[:, :, rows], Z[:, :, rows], H[:, :, rows]
    else:
        P = pd.cpu().numpy()
        nbad = p_mismatch(P, ref.p)
        assert nbad == 0, f"{nbad} P codes differ, first at {np.argwhere(P != ref.p)[:5]}"
    assert np.array_equal(Z, ref.row_zeros)
    assert np.array_equal(H, oracle.row_hash(ref.p))
    err = max_head_rel(o, ref.out)
    assert err <= TOL_O, err
    return out


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("cond", list(synth.CONDITIONS))
def test_int8_qwen_like_ragged(pan, d, cond):
    w = synth.qwen_like(1, 6, 2, d, seed=610 + d, N=300, texts=2)
    run_int8(pan, w, cond)


@pytest.mark.parametrize("p_scale", [1.0, 256.0, 448.0])
@pytest.mark.parametrize("kv_order", [0, 1])
@pytest.mark.parametrize("block_n", [64, 128])
def test_int8_scales_orders_blocks(pan, p_scale, kv_order, block_n):
    w = synth.qwen_like(1, 4, 1, 128, seed=630, N=420, texts=1)
    run_int8(pan, w, "rotated", p_scale, kv_order, block_n)


@pytest.mark.parametrize("N", [1, 127, 128, 129])
def test_int8_degenerate_lengths(pan, N):
    w = synth.qwen_like(1, 2, 1, 64, seed=640 + N, N=N, texts=1)
    for cond in ("plain", "centered_rotated"):
        run_int8(pan, w, cond)


@pytest.mark.parametrize("causal", [False, True])
def test_int8_sink_heads(pan, causal):
    w = synth.long_context(seed=650, N=384, hq=4, hkv=2, d=128, delta=8.0)
    for cond in ("rotated", "centered_rotated"):
        run_int8(pan, w, cond, causal=causal)


@pytest.mark.timeout(600)
def test_int8_long_context_full_size(pan):
    """The 32k-token workload in the benchmark's launch (centered_rotated):
    prologue bit-exact in full; outputs, checksums and underflow counts on the
    first, middle and last 64 rows of every head."""
    w = synth.long_context()
    rows = np.concatenate([np.arange(0, 64), np.arange(16384, 16448), np.arange(32704, 32768)]).astype(np.int32)
    run_int8(pan, w, "centered_rotated", rows=rows)
