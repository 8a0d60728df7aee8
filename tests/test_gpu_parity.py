"""GPU parity: the HIP path (through the C ABI) against the oracle.

Bars: E4M3 codes of Q/K/V and of P~ bit-exact; outputs within 2e-3 relative
Frobenius error per head of the emulator's binary32 result; per-head errors of
the HIP reduction within 1e-12 (relative) of the oracle's metric."""
import math

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


def run_case(pan, w, cond, p_scale, kv_order, block_n, causal, rows=None, check_ideal=False):
    flags = synth.CONDITIONS[cond]
    B, hq, N, d = w.q.shape
    hkv = w.k.shape[1]
    pipe = pan.AttnPipeline(B, hq, hkv, N, d)
    q, k, v = dev(w.q, w.dtype), dev(w.k, w.dtype), dev(w.v, w.dtype)
    print(f"case {w.name} {cond} S={p_scale} order={kv_order} bc={block_n} causal={causal} shape={w.q.shape}", flush=True)
    gp = pipe.prepare(q, k, v, signs=signs_dev(w), **flags)
    op = oracle.prepare(w.q, w.k, w.v, signs=w.signs, **flags)
    torch.cuda.synchronize()
    compare_prepared(gp, op, N, flags["center"])
    pd = torch.zeros((B, hq, N, N), dtype=torch.uint8, device="cuda")
    rz = torch.zeros((B, hq, N), dtype=torch.int32, device="cuda")
    rh = torch.zeros((B, hq, N), dtype=torch.int64, device="cuda")
    out = pipe.fwd(gp, p_scale=p_scale, kv_order=kv_order, block_n=block_n, causal=causal, p_dump=pd, row_hash=rh,
                   row_zeros=rz, k_sink=4)
    out_nodump = pipe.fwd(gp, p_scale=p_scale, kv_order=kv_order, block_n=block_n, causal=causal)
    torch.cuda.synchronize()
    ref = oracle.attention_fp8(op, p_scale=p_scale, kv_order=kv_order, block_n=block_n, causal=causal,
                               rows=rows, want_p=True, k_sink=4)
    o = out.cpu().numpy()
    assert np.array_equal(o, out_nodump.cpu().numpy()), "dump and timed variants differ"
    P = pd.cpu().numpy()
    Z = rz.cpu().numpy().astype(np.uint32)
    H = rh.cpu().numpy().view(np.uint64)
    if rows is not None:
        o, P, Z, H = o[:, :, rows], P[:, :, rows], Z[:, :, rows], H[:, :, rows]
    nbad = p_mismatch(P, ref.p)
    assert nbad == 0, f"{nbad} P codes differ, first at {np.argwhere(P != ref.p)[:5]}"
    assert np.array_equal(Z, ref.row_zeros)
    assert np.array_equal(H, oracle.row_hash(ref.p)), "P row checksums differ"
    err = max_head_rel(o, ref.out)
    assert err <= TOL_O, err
    if check_ideal:
        ideal = oracle.attention_f64(w.q, w.k, w.v, causal=causal, rows=rows)
        ideal_dev = torch.from_numpy(ideal).cuda()
        rows_dev = None if rows is None else torch.from_numpy(np.asarray(rows, np.int32)).cuda()
        rel = pipe.head_error(out, ideal_dev, rows=rows_dev).cpu().numpy()
        ref_rel = oracle.head_errors(o, ideal).ravel()
        np.testing.assert_allclose(rel, ref_rel, rtol=1e-12, atol=0)
        return rel
    return None


@pytest.mark.parametrize("cond", list(synth.CONDITIONS))
def test_illustration_all_conditions(pan, cond):
    """Single head, N=256, d=64, shared key of norm 20; S=256, forward, block 64."""
    w = synth.illustration()
    rel = run_case(pan, w, cond, 256.0, 0, 64, True, check_ideal=True)
    print(cond, "log1p(rel err vs fp64) =", np.log1p(rel))


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("cond", list(synth.CONDITIONS))
def test_qwen_like_ragged(pan, d, cond):
    """BF16 RoPE'd operands with outlier channels and a shared key vector,
    GQA, N = 300 (three 128-token tiles with a ragged tail)."""
    w = synth.qwen_like(1, 6, 2, d, seed=210 + d, N=300, texts=2)
    run_case(pan, w, cond, 256.0, 1, 128, True, check_ideal=True)


@pytest.mark.parametrize("p_scale", [1.0, 2.0, 64.0, 256.0, 448.0])
@pytest.mark.parametrize("kv_order", [0, 1])
@pytest.mark.parametrize("block_n", [64, 128])
def test_scales_orders_blocks(pan, p_scale, kv_order, block_n):
    w = synth.qwen_like(1, 4, 1, 128, seed=230, N=200, texts=1)
    run_case(pan, w, "rotated", p_scale, kv_order, block_n, True)


@pytest.mark.parametrize("causal", [False, True])
def test_noncausal_and_sinks(pan, causal):
    w = synth.long_context(seed=401, N=384, hq=4, hkv=2, d=128, delta=8.0)
    for cond in ("rotated", "centered_rotated"):
        run_case(pan, w, cond, 256.0, 1, 128, causal, check_ideal=True)


@pytest.mark.parametrize("N", [1, 2, 127, 128, 129])
def test_degenerate_lengths(pan, N):
    w = synth.qwen_like(1, 2, 1, 64, seed=240 + N, N=N, texts=1)
    for cond in synth.CONDITIONS:
        run_case(pan, w, cond, 256.0, 1, 128, True)


def test_mean_key_tree_with_padding(pan):
    """41 chunks of 64 tokens (the last one ragged): the chunk tree is padded
    to 64 leaves and split over the reduction's workers."""
    w = synth.qwen_like(1, 2, 1, 64, seed=245, N=40 * 64 + 17, texts=1)
    for cond in ("centered", "centered_rotated"):
        run_case(pan, w, cond, 256.0, 1, 128, True)


def test_zero_head_and_strided_input(pan):
    """An all-zero head gets unit scales; a strided [B,N,H,d] view quantises
    exactly like the dense copy."""
    w = synth.qwen_like(1, 4, 2, 128, seed=250, N=256, texts=1)
    w.q[0, 1] = 0.0
    w.v[0, 0] = 0.0
    run_case(pan, w, "centered_rotated", 256.0, 1, 128, True)
    B, hq, N, d = w.q.shape
    hkv = w.k.shape[1]
    pipe = pan.AttnPipeline(B, hq, hkv, N, d)
    qd, kd, vd = dev(w.q, "bf16"), dev(w.k, "bf16"), dev(w.v, "bf16")
    qs = qd.transpose(1, 2).contiguous().transpose(1, 2)   # [B,H,N,d] view of [B,N,H,d] storage
    ks = kd.transpose(1, 2).contiguous().transpose(1, 2)
    vs = vd.transpose(1, 2).contiguous().transpose(1, 2)
    a = pipe.prepare(qd, kd, vd, rotate=True, center=True, signs=signs_dev(w))
    b = pipe.prepare(qs, ks, vs, rotate=True, center=True, signs=signs_dev(w))
    torch.cuda.synchronize()
    for x, y in ((a.q8, b.q8), (a.k8, b.k8), (a.v8t, b.v8t), (a.q_desc, b.q_desc), (a.k_desc, b.k_desc)):
        assert torch.equal(x, y)


def test_nonfinite_input_flagged(pan):
    w = synth.qwen_like(1, 2, 1, 64, seed=260, N=64, texts=1)
    w.k[0, 0, 5, 3] = np.inf
    pipe = pan.AttnPipeline(1, 2, 1, 64, 64)
    gp = pipe.prepare(dev(w.q, "bf16"), dev(w.k, "bf16"), dev(w.v, "bf16"), rotate=False, center=False)
    torch.cuda.synchronize()
    assert int(gp.status.cpu()[0]) & 1


@pytest.mark.parametrize("delta", [0.0, 7.0, 12.0])
def test_pcast_sweep_points(pan, delta):
    """P-collapse sweep point (N=4096, d=128, non-causal, FP32 operands, only P
    cast): every grid setting, sampled rows against the oracle."""
    w = synth.pcast_sweep(delta)
    rows = np.arange(0, 4096, 31)
    pipe = pan.AttnPipeline(1, 1, 1, 4096, 128)
    q, k, v = dev(w.q, "f32"), dev(w.k, "f32"), dev(w.v, "f32")
    for order in (0, 1):
        for S in (1.0, 256.0, 448.0):
            print(f"pcast delta={delta} order={order} S={S}", flush=True)
            pd = torch.zeros((1, 1, 4096, 4096), dtype=torch.uint8, device="cuda")
            rz = torch.zeros((1, 1, 4096), dtype=torch.int32, device="cuda")
            rh = torch.zeros((1, 1, 4096), dtype=torch.int64, device="cuda")
            out = pipe.fwd_f32(q, k, v, p_scale=S, kv_order=order, block_n=128, causal=False, p_dump=pd,
                               row_hash=rh, row_zeros=rz, k_sink=4)
            torch.cuda.synchronize()
            ref = oracle.attention_pcast_f32(w.q, w.k, w.v, p_scale=S, kv_order=order, block_n=128, causal=False,
                                             rows=rows, want_p=True, k_sink=4)
            P = pd.cpu().numpy()[:, :, rows]
            assert p_mismatch(P, ref.p) == 0
            assert np.array_equal(rz.cpu().numpy()[:, :, rows].astype(np.uint32), ref.row_zeros)
            assert np.array_equal(rh.cpu().numpy().view(np.uint64)[:, :, rows], oracle.row_hash(ref.p))
            assert max_head_rel(out.cpu().numpy()[:, :, rows], ref.out) <= TOL_O


def test_lse_matches_ideal_logsumexp(pan):
    """Natural-log sum-exp of the scaled logits (without centring, which shifts
    every logit of a row by q.mean_k) near the binary64 value of the original
    operands (E4M3 rounding of Q and K moves the logits by a few percent)."""
    w = synth.qwen_like(1, 2, 1, 128, seed=270, N=256, texts=1)
    B, hq, N, d = w.q.shape
    pipe = pan.AttnPipeline(B, hq, 1, N, d)
    gp = pipe.prepare(dev(w.q, "bf16"), dev(w.k, "bf16"), dev(w.v, "bf16"), rotate=True, center=False,
                      signs=signs_dev(w))
    lse = torch.empty((B, hq, N), dtype=torch.float32, device="cuda")
    pipe.fwd(gp, lse=lse)
    torch.cuda.synchronize()
    z = np.einsum("bhnd,bhmd->bhnm", w.q.astype(np.float64), np.repeat(w.k, hq, 1).astype(np.float64)) / math.sqrt(d)
    z = np.where(np.tril(np.ones((N, N), bool)), z, -np.inf)
    ref = np.log(np.exp(z - z.max(-1, keepdims=True)).sum(-1)) + z.max(-1)
    assert np.abs(lse.cpu().numpy() - ref).max() < 0.05 * np.abs(ref).max() + 0.05


LSE_TOL = 3e-6


@pytest.mark.parametrize("variant", ["per_head", "tiles", "int8"])
@pytest.mark.parametrize("d,bn", [(128, 128), (128, 64), (64, 128), (64, 64)])
@pytest.mark.parametrize("order", [0, 1])
def test_lse_matches_the_emulator(pan, variant, d, bn, order):
    """The LSE output against the emulator's (m*c + log2 l) * ln 2 from its own
    running max and row sum: equal to binary32 rounding of l and of the final
    sum (|diff| <= 3e-6 * max(1, |lse|)), on every kernel that writes it
    (pipelined, block-64 and head_dim-64 forms; per-tile scales; int8 scores)."""
    w = synth.qwen_like(1, 4, 2, d, seed=280 + d + bn + order, N=333, texts=1)
    B, hq, N, _ = w.q.shape
    pipe = pan.AttnPipeline(B, hq, 2, N, d)
    flags = dict(rotate=True, center=True, tiles=variant == "tiles", int8=variant == "int8")
    gp = pipe.prepare(dev(w.q, "bf16"), dev(w.k, "bf16"), dev(w.v, "bf16"), signs=signs_dev(w), **flags)
    op = oracle.prepare(w.q, w.k, w.v, signs=w.signs, **flags)
    for causal in (True, False):
        lse = torch.empty((B, hq, N), dtype=torch.float32, device="cuda")
        pipe.fwd(gp, p_scale=256.0, kv_order=order, block_n=bn, causal=causal, lse=lse)
        torch.cuda.synchronize()
        ref = oracle.attention_fp8(op, p_scale=256.0, kv_order=order, block_n=bn, causal=causal).lse
        got = lse.cpu().numpy().astype(np.float64)
        err = np.abs(got - ref) / np.maximum(1.0, np.abs(ref))
        assert err.max() <= LSE_TOL, (causal, err.max(), np.unravel_index(err.argmax(), err.shape))


def test_lse_matches_the_emulator_pcast_f32(pan):
    """The binary32 P-cast-only path's LSE against the emulator's."""
    w = synth.pcast_sweep(7.0, N=1024)
    B, hq, N, d = w.q.shape
    pipe = pan.AttnPipeline(B, hq, hq, N, d)
    q, k, v = (torch.from_numpy(x).cuda() for x in (w.q, w.k, w.v))
    rows = np.arange(0, N, 37, dtype=np.int32)
    for order in (0, 1):
        lse = torch.empty((B, hq, N), dtype=torch.float32, device="cuda")
        pipe.fwd_f32(q, k, v, p_scale=256.0, kv_order=order, block_n=128, causal=False, lse=lse)
        torch.cuda.synchronize()
        ref = oracle.attention_pcast_f32(w.q, w.k, w.v, p_scale=256.0, kv_order=order, block_n=128, causal=False,
                                         rows=rows).lse
        got = lse.cpu().numpy()[:, :, rows].astype(np.float64)
        err = np.abs(got - ref) / np.maximum(1.0, np.abs(ref))
        assert err.max() <= LSE_TOL, (order, err.max())


def test_abi_rejects_bad_arguments(pan):
    pipe = pan.AttnPipeline(1, 2, 1, 128, 64)
    q = torch.zeros((1, 2, 128, 64), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((1, 1, 128, 64), dtype=torch.bfloat16, device="cuda")
    gp = pipe.prepare(q, k, k, rotate=False, center=False)
    for kw, status in ((dict(block_n=96), -4), (dict(kv_order=2), -4), (dict(p_scale=100.0), -3),
                       (dict(p_scale=0.0), -4), (dict(p_scale=512.0), -4), (dict(softmax_scale=-1.0), -4)):
        with pytest.raises(pan.Fp8AttnError) as e:
            pipe.fwd(gp, **kw)
        assert e.value.status == status, kw
    with pytest.raises(pan.Fp8AttnError) as e:
        pipe.prepare(q, k, k, rotate=True, center=False, signs=None)
    assert e.value.status == -1
    torch.cuda.synchronize()
