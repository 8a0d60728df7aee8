"""GPU parity of the per-tile Q/K scaling variant (one max-based scale per
128-token tile of a head instead of per (batch, head); V per head): the
prologue's codes and tile descales bit-exact against the oracle, every P~
code and underflow count bit-exact, the P~ row checksums equal, outputs within
2e-3 per head of the oracle's, and the dump variant equal to the timed one."""
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


def run_tiles(pan, w, cond, p_scale=256.0, kv_order=1, block_n=128, causal=True, rows=None, prefix=False):
    flags = synth.CONDITIONS[cond]
    B, hq, N, d = w.q.shape
    hkv = w.k.shape[1]
    pipe = pan.AttnPipeline(B, hq, hkv, N, d)
    print(f"tiles {w.name} {cond} S={p_scale} order={kv_order} bc={block_n} causal={causal} shape={w.q.shape}",
          flush=True)
    gp = pipe.prepare(dev(w.q, w.dtype), dev(w.k, w.dtype), dev(w.v, w.dtype), signs=signs_dev(w), tiles=True,
                      prefix=prefix, **flags)
    op = oracle.prepare(w.q, w.k, w.v, signs=w.signs, tiles=True, prefix=prefix, **flags)
    torch.cuda.synchronize()
    compare_prepared(gp, op, N, flags["center"])
    kw = dict(p_scale=p_scale, kv_order=kv_order, block_n=block_n, causal=causal)
    pd = torch.zeros((B, hq, N, N), dtype=torch.uint8, device="cuda")
    rz = torch.zeros((B, hq, N), dtype=torch.int32, device="cuda")
    rh = torch.zeros((B, hq, N), dtype=torch.int64, device="cuda")
    out = pipe.fwd(gp, p_dump=pd, row_hash=rh, row_zeros=rz, k_sink=4, **kw)
    out_nodump = pipe.fwd(gp, **kw)
    torch.cuda.synchronize()
    ref = oracle.attention_fp8(op, rows=rows, want_p=True, k_sink=4, **kw)
    o = out.cpu().numpy()
    assert np.array_equal(o, out_nodump.cpu().numpy()), "dump and timed variants differ"
    P, Z = pd.cpu().numpy(), rz.cpu().numpy().astype(np.uint32)
    H = rh.cpu().numpy().view(np.uint64)
    if rows is not None:
        o, P, Z, H = o[:, :, rows], P[:, :, rows], Z[:, :, rows], H[:, :, rows]
    nbad = p_mismatch(P, ref.p)
    assert nbad == 0, f"{nbad} P codes differ, first at {np.argwhere(P != ref.p)[:5]}"
    assert np.array_equal(Z, ref.row_zeros)
    assert np.array_equal(H, oracle.row_hash(ref.p))
    assert max_head_rel(o, ref.out) <= TOL_O
    return out, gp


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("cond", list(synth.CONDITIONS))
def test_tiles_qwen_like_ragged(pan, d, cond):
    w = synth.qwen_like(1, 6, 2, d, seed=510 + d, N=300, texts=2)
    run_tiles(pan, w, cond)


@pytest.mark.parametrize("p_scale", [1.0, 256.0, 448.0])
@pytest.mark.parametrize("kv_order", [0, 1])
@pytest.mark.parametrize("block_n", [64, 128])
def test_tiles_scales_orders_blocks(pan, p_scale, kv_order, block_n):
    w = synth.qwen_like(1, 4, 1, 128, seed=530, N=420, texts=1)
    run_tiles(pan, w, "rotated", p_scale, kv_order, block_n)


@pytest.mark.parametrize("N", [1, 127, 128, 129, 257])
def test_tiles_degenerate_lengths(pan, N):
    w = synth.qwen_like(1, 2, 1, 64, seed=540 + N, N=N, texts=1)
    for cond in ("plain", "centered_rotated"):
        run_tiles(pan, w, cond)


@pytest.mark.parametrize("causal", [True, False])
def test_tiles_of_very_different_magnitude(pan, causal):
    """Tile magnitudes 1, 16, 1/8, 4 (Q) and shifted by one tile (K): the tile
    descales differ by up to 128x, so a wrong tile anywhere shows."""
    w = synth.qwen_like(1, 4, 2, 128, seed=550, N=512, texts=1)
    gains = (1.0, 16.0, 0.125, 4.0)
    for t in range(4):
        w.q[:, :, 128 * t:128 * (t + 1)] *= np.float32(gains[t])
        w.k[:, :, 128 * t:128 * (t + 1)] *= np.float32(gains[(t + 1) % 4])
    for cond in ("plain", "rotated"):
        run_tiles(pan, w, cond, causal=causal)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("cond", list(synth.CONDITIONS))
def test_prefix_scales(pan, d, cond):
    """Prefix tile scales (tile t from the largest maximum of tiles 0..t) on
    tiles of rising and falling magnitude; centred conditions take the mean key
    over the first tile only (the mean is compared bit for bit)."""
    w = synth.qwen_like(1, 4, 2, d, seed=570 + d, N=650, texts=1)
    gains = (0.5, 4.0, 1.0, 0.25, 8.0, 2.0)
    for t in range(6):
        w.q[:, :, 128 * t:128 * (t + 1)] *= np.float32(gains[t])
        w.k[:, :, 128 * t:128 * (t + 1)] *= np.float32(gains[(t + 2) % 6])
    run_tiles(pan, w, cond, prefix=True)
    run_tiles(pan, w, cond, kv_order=0, block_n=64, causal=False, prefix=True)


@pytest.mark.parametrize("center", [False, True])
def test_prefix_scales_ignore_future_tokens(pan, center):
    """Changing tokens from tile 2 on leaves tiles 0 and 1's codes and scales
    (and, centred, the mean key) as they were."""
    import precision_attention_numerics_amd as pan_
    w = synth.qwen_like(1, 2, 1, 128, seed=580, N=512, texts=1)
    pipe = pan_.AttnPipeline(1, 2, 1, 512, 128)
    args = dict(rotate=True, center=center, signs=signs_dev(w), tiles=True, prefix=True)
    a = pipe.prepare(dev(w.q, "bf16"), dev(w.k, "bf16"), dev(w.v, "bf16"), **args)
    q2, k2 = w.q.copy(), w.k.copy()
    q2[:, :, 256:] *= np.float32(8.0)
    k2[:, :, 300:] += np.float32(5.0)
    b = pipe.prepare(dev(q2, "bf16"), dev(k2, "bf16"), dev(w.v, "bf16"), **args)
    torch.cuda.synchronize()
    assert torch.equal(a.q8[:, :, :256], b.q8[:, :, :256]) and torch.equal(a.k8[:, :, :256], b.k8[:, :, :256])
    qa, qb = a.q_desc.view(2, 4), b.q_desc.view(2, 4)
    assert torch.equal(qa[:, :2], qb[:, :2]) and torch.equal(a.k_desc[:2], b.k_desc[:2])
    if center:
        assert torch.equal(a.k_mean, b.k_mean)


def test_equal_tile_maxima_match_the_per_head_kernel(pan):
    """Every tile holds the same largest magnitude: the tile-scaled forward must
    give the per-head forward's output bit for bit."""
    N = 512
    w = synth.qwen_like(1, 4, 1, 128, seed=560, N=N, texts=1)
    q, k = np.clip(w.q, -2.0, 2.0), np.clip(w.k, -2.0, 2.0)
    for t in range(N // 128):
        q[:, :, 128 * t, 5] = 3.0
        k[:, :, 128 * t + 2, 9] = -3.0
    w.q, w.k = q, k
    out_t, _ = run_tiles(pan, w, "plain")
    pipe = pan.AttnPipeline(1, 4, 1, N, 128)
    gp = pipe.prepare(dev(w.q, w.dtype), dev(w.k, w.dtype), dev(w.v, w.dtype), rotate=False, center=False)
    out_h = pipe.fwd(gp, p_scale=256.0, kv_order=1, block_n=128, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(out_t, out_h)


@pytest.mark.timeout(600)
def test_tiles_long_context_full_size(pan):
    """The 32k-token workload with per-tile scales (centered_rotated, the
    benchmark's launch): prologue bit-exact in full, outputs and P~ codes on the
    first, middle and last 64 rows of every head."""
    w = synth.long_context()
    rows = np.concatenate([np.arange(0, 64), np.arange(16384, 16448), np.arange(32704, 32768)]).astype(np.int32)
    B, hq, N, d = w.q.shape
    hkv = w.k.shape[1]
    flags = synth.CONDITIONS["centered_rotated"]
    pipe = pan.AttnPipeline(B, hq, hkv, N, d)
    gp = pipe.prepare(dev(w.q, w.dtype), dev(w.k, w.dtype), dev(w.v, w.dtype), signs=signs_dev(w), tiles=True,
                      **flags)
    op = oracle.prepare(w.q, w.k, w.v, signs=w.signs, tiles=True, **flags)
    torch.cuda.synchronize()
    compare_prepared(gp, op, N, True)
    kw = dict(p_scale=256.0, kv_order=1, block_n=128, causal=True)
    out = pipe.fwd(gp, **kw)
    rows_dev = torch.from_numpy(rows).long().cuda()
    rh = torch.zeros((B, hq, N), dtype=torch.int64, device="cuda")
    out_d = pipe.fwd(gp, row_hash=rh, **kw)
    torch.cuda.synchronize()
    assert torch.equal(out, out_d)
    ref = oracle.attention_fp8(op, rows=rows, want_p=True, **kw)
    assert max_head_rel(out[:, :, rows_dev].cpu().numpy(), ref.out) <= TOL_O
    assert np.array_equal(rh[:, :, rows_dev].cpu().numpy().view(np.uint64), oracle.row_hash(ref.p))
