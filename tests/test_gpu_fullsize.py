"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times (S = 256, reverse KV order, KV block 128, causal).

Long context (batch 1, 32 query / 8 KV heads, d = 128, N = 32768): the
prologue is compared bit-exactly in full; the timed (non-dump) forward is
checked against the emulator on the first, middle and last 128-row query tile
of every head plus 128 rows spread over the sequence; then each head is run
again alone with the P~ dump on views of the same prepared codes, its output
must equal the full run's head bit for bit, and the sampled rows' P~ codes and
zero counts must equal the oracle's.

Qwen2.5-0.5B / 1.5B shapes (24 / 28 layers x 3 texts, N = 1024): the prologue
bit-exactly in full and the forward of the whole stack in one launch; then,
layer by layer, the per-head outputs against the emulator and the layer's full
P~ dump (run on views of that layer's codes) against the oracle's."""
import time

import numpy as np
import pytest
import torch

import oracle
import synth
from _gpu_helpers import compare_prepared, dev, max_head_rel, p_mismatch, signs_dev

pytestmark = pytest.mark.gpu
TOL_O = 2e-3
K_SINK = 4
ROW_TILES = ((0, 128), (16384, 16512), (32640, 32768))


@pytest.fixture(scope="module")
def pan():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    import precision_attention_numerics_amd as pan
    return pan


@pytest.fixture(scope="module")
def workloads():
    cache = {}

    def get(name):
        if name not in cache:
            t = time.time()
            cache[name] = getattr(synth, name)()
            print(f"[fullsize] generated {name} {cache[name].q.shape} in {time.time() - t:.1f}s", flush=True)
        return cache[name]
    return get


def _head_view(pan, gp, b0, b1, h0, h1, hkv0, hkv1, hq, hkv):
    """Prepared views of batches [b0,b1) and heads [h0,h1) / KV heads [hkv0,hkv1);
    valid as one contiguous operand only when either the batch or the head
    range is a single entry spanning the whole other axis."""
    return pan.Prepared(gp.q8[b0:b1, h0:h1], gp.k8[b0:b1, hkv0:hkv1], gp.v8t[b0:b1, hkv0:hkv1],
                        gp.q_desc.view(-1, hq)[b0:b1, h0:h1].reshape(-1),
                        gp.k_desc.view(-1, hkv)[b0:b1, hkv0:hkv1].reshape(-1),
                        gp.v_desc.view(-1, hkv)[b0:b1, hkv0:hkv1].reshape(-1), gp.k_mean, gp.status)


def _prepare_both(pan, w, cond):
    flags = synth.CONDITIONS[cond]
    B, hq, N, d = w.q.shape
    hkv = w.k.shape[1]
    pipe = pan.AttnPipeline(B, hq, hkv, N, d)
    t = time.time()
    gp = pipe.prepare(dev(w.q, w.dtype), dev(w.k, w.dtype), dev(w.v, w.dtype), signs=signs_dev(w), **flags)
    op = oracle.prepare(w.q, w.k, w.v, signs=w.signs, **flags)
    torch.cuda.synchronize()
    compare_prepared(gp, op, N, flags["center"])
    print(f"[fullsize] {w.name} {cond}: prologue bit-exact ({time.time() - t:.1f}s)", flush=True)
    return pipe, gp, op


@pytest.mark.timeout(900)
@pytest.mark.parametrize("cond", ["centered_rotated", "rotated"])
def test_long_context_full_size(pan, workloads, cond):
    w = workloads("long_context")
    B, hq, N, d = w.q.shape
    hkv = w.k.shape[1]
    grp = hq // hkv
    pipe, gp, op = _prepare_both(pan, w, cond)
    kw = dict(p_scale=w.p_scale, kv_order=w.kv_order, block_n=w.block_n, causal=True)
    out = pipe.fwd(gp, **kw)
    spread = np.arange(128) * (N // 128) + (np.arange(128) * 37) % (N // 128)
    rows = np.unique(np.concatenate([np.arange(a, b) for a, b in ROW_TILES] + [spread])).astype(np.int32)
    rows_dev = torch.from_numpy(rows).long().cuda()
    o_rows = out[:, :, rows_dev].cpu().numpy()
    t = time.time()
    ref = oracle.attention_fp8(op, rows=rows, want_p=True, k_sink=K_SINK, **kw)
    print(f"[fullsize] oracle on {rows.size} rows x {hq} heads: {time.time() - t:.1f}s", flush=True)
    errs = oracle.head_errors(o_rows, ref.out)
    assert max_head_rel(o_rows, ref.out) <= TOL_O, errs.max()
    print(f"[fullsize] sampled-row error vs emulator: max {errs.max():.3e}", flush=True)

    sub = pan.AttnPipeline(1, 1, 1, N, d)
    pd = torch.empty((1, 1, N, N), dtype=torch.uint8, device="cuda")
    rz = torch.empty((1, 1, N), dtype=torch.int32, device="cuda")
    rh = torch.empty((1, 1, N), dtype=torch.int64, device="cuda")
    for h in range(hq):
        g = h // grp
        pd.zero_()
        rz.zero_()
        oh = sub.fwd(_head_view(pan, gp, 0, 1, h, h + 1, g, g + 1, hq, hkv), p_dump=pd, row_hash=rh,
                     row_zeros=rz, k_sink=K_SINK, **kw)
        torch.cuda.synchronize()
        assert torch.equal(oh[0, 0], out[0, h]), f"head {h}: single-head dump run differs from the full run"
        P = pd[0, 0][rows_dev].cpu().numpy()
        nbad = p_mismatch(P, ref.p[0, h])
        assert nbad == 0, f"head {h}: {nbad} P codes differ, first at {np.argwhere(P != ref.p[0, h])[:5]}"
        Z = rz[0, 0][rows_dev].cpu().numpy().astype(np.uint32)
        assert np.array_equal(Z, ref.row_zeros[0, h]), f"head {h}: zero counts differ"
        Hs = rh[0, 0][rows_dev].cpu().numpy().view(np.uint64)
        assert np.array_equal(Hs, oracle.row_hash(ref.p[0, h])), f"head {h}: row checksums differ"
    print(f"[fullsize] {cond}: P codes of {rows.size} rows x {hq} heads bit-exact", flush=True)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("cond", list(synth.CONDITIONS))
@pytest.mark.parametrize("model", ["qwen05b", "qwen15b"])
def test_qwen_stack_full_shape(pan, workloads, model, cond):
    w = workloads(model)
    B, hq, N, d = w.q.shape
    hkv = w.k.shape[1]
    texts, layers = w.meta["texts"], w.meta["layers"]
    pipe, gp, op = _prepare_both(pan, w, cond)
    kw = dict(p_scale=w.p_scale, kv_order=w.kv_order, block_n=w.block_n, causal=True)
    out = pipe.fwd(gp, **kw)
    torch.cuda.synchronize()
    sub = pan.AttnPipeline(texts, hq, hkv, N, d)
    pd = torch.empty((texts, hq, N, N), dtype=torch.uint8, device="cuda")
    rz = torch.empty((texts, hq, N), dtype=torch.int32, device="cuda")
    rh = torch.empty((texts, hq, N), dtype=torch.int64, device="cuda")
    worst = 0.0
    t0 = time.time()
    for layer in range(layers):
        b0, b1 = layer * texts, (layer + 1) * texts
        ol = oracle.Prepared(op.q8[b0:b1], op.k8[b0:b1], op.v8[b0:b1], op.q_desc[b0:b1], op.k_desc[b0:b1],
                             op.v_desc[b0:b1], None if op.k_mean is None else op.k_mean[b0:b1])
        t = time.time()
        ref = oracle.attention_fp8(ol, want_p=True, k_sink=K_SINK, **kw)
        o = out[b0:b1].cpu().numpy()
        errs = oracle.head_errors(o, ref.out)
        assert max_head_rel(o, ref.out) <= TOL_O, errs.max()
        pd.zero_()
        rz.zero_()
        ol_dev = sub.fwd(_head_view(pan, gp, b0, b1, 0, hq, 0, hkv, hq, hkv), p_dump=pd, row_hash=rh,
                         row_zeros=rz, k_sink=K_SINK, **kw)
        torch.cuda.synchronize()
        assert torch.equal(ol_dev, out[b0:b1]), f"layer {layer}: dump run differs from the full run"
        P = pd.cpu().numpy()
        nbad = p_mismatch(P, ref.p)
        assert nbad == 0, f"layer {layer}: {nbad} P codes differ, first at {np.argwhere(P != ref.p)[:5]}"
        assert np.array_equal(rz.cpu().numpy().astype(np.uint32), ref.row_zeros), f"layer {layer}: zero counts"
        assert np.array_equal(rh.cpu().numpy().view(np.uint64), oracle.row_hash(ref.p)), f"layer {layer}: checksums"
        worst = max(worst, float(errs.max()))
        if layer % 8 == 0:
            print(f"[fullsize] {w.name} {cond} layer {layer}: P bit-exact ({time.time() - t:.1f}s)", flush=True)
    print(f"[fullsize] {w.name} {cond}: {layers} layers, P bit-exact, max head error {worst:.3e} "
          f"({time.time() - t0:.1f}s)", flush=True)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("N", [1 << 18, 1 << 20])
def test_very_long_sequence_sampled(pan, N):
    """One KV head with two query heads at N = 262144 and 1048576 (8 and 32
    times the benchmark's length; up to 8192 KV blocks per row) in the
    benchmark's launch:
    prologue bit-exact in full; on the first, middle and last 128-row query
    tile plus 64 rows spread over the sequence, the output within 2e-3 per
    head of the emulator and the per-row P~ checksums and underflow counts
    equal to the oracle's (a full P~ dump would be 2 x N^2 bytes)."""
    w = synth.long_context(seed=410, N=N, hq=2, hkv=1)
    B, hq, _, d = w.q.shape
    cond = "centered_rotated"
    pipe, gp, op = _prepare_both(pan, w, cond)
    kw = dict(p_scale=w.p_scale, kv_order=w.kv_order, block_n=w.block_n, causal=True)
    rz = torch.zeros((B, hq, N), dtype=torch.int32, device="cuda")
    rh = torch.zeros((B, hq, N), dtype=torch.int64, device="cuda")
    out = pipe.fwd(gp, row_hash=rh, row_zeros=rz, k_sink=K_SINK, **kw)
    out_timed = pipe.fwd(gp, **kw)
    torch.cuda.synchronize()
    spread = np.arange(64) * (N // 64) + (np.arange(64) * 97) % (N // 64)
    tiles = [np.arange(0, 128), np.arange(N // 2, N // 2 + 128), np.arange(N - 128, N)]
    rows = np.unique(np.concatenate(tiles + [spread])).astype(np.int32)
    rows_dev = torch.from_numpy(rows).long().cuda()
    assert torch.equal(out[:, :, rows_dev], out_timed[:, :, rows_dev]), "checksum and timed variants differ"
    t = time.time()
    ref = oracle.attention_fp8(op, rows=rows, want_p=True, k_sink=K_SINK, **kw)
    print(f"[fullsize] N={N}: oracle on {rows.size} rows x {hq} heads: {time.time() - t:.1f}s", flush=True)
    o = out[:, :, rows_dev].cpu().numpy()
    assert max_head_rel(o, ref.out) <= TOL_O
    Z = rz[:, :, rows_dev].cpu().numpy().astype(np.uint32)
    assert np.array_equal(Z, ref.row_zeros), "underflow counts differ"
    H = rh[:, :, rows_dev].cpu().numpy().view(np.uint64)
    assert np.array_equal(H, oracle.row_hash(ref.p)), "row checksums differ"
    print(f"[fullsize] N={N}: {rows.size} rows x {hq} heads: checksums and underflow counts equal, "
          f"max head error {oracle.head_errors(o, ref.out).max():.2e}", flush=True)
