"""GPU test of the exp fix-up: inputs built so that some key's exponent x equals
exactly one of the binary32 values where the hardware exp2 would round the
other way, in a masked (diagonal) and an unmasked block; every P code must
still equal the oracle's (which uses the correctly rounded 2^x), and the
timed variant (no dump) must return the dump variant's output bit for bit.

Construction: Q rows are (448, 0, ..., 0) and K rows (a_j, 0, ..., 0) with a_j
E4M3 values and max 448, so the codes are exact, both descales are 1 and each
score is the single exact product 448*a_j.  Then c = RN32(scale*log2 e) and
x_j = fma(448*a_j, c, -RN32(448*448*c)); the softmax scale is searched over
consecutive binary32 values until x_j hits the target bit pattern."""
import numpy as np
import pytest
import torch

import oracle
from _gpu_helpers import p_mismatch

pytestmark = pytest.mark.gpu

LOG2E = 1.4426950408889634
TARGETS = {256.0: (0xBD3B9CB2, 0xBEF3EFB2), 448.0: (0xBF5A689A, 0xBFED344D)}
E4M3_VALUES = np.array([(1 + m / 8) * 2.0 ** e for e in range(-6, 9) for m in range(8) if (1 + m / 8) * 2.0 ** e <= 448])


def find_scale(target_bits: int):
    """(softmax_scale, a) with fma(448 a, c, -RN32(448*448 c)) == target exactly."""
    tx = float(np.uint32(target_bits).view(np.float32))
    smax = 448.0 * 448.0
    for a in sorted(E4M3_VALUES, reverse=True):
        if a >= 448:
            continue
        ds = smax - 448.0 * a
        c0 = -tx / ds
        scale0 = np.float32(c0 / LOG2E)
        base = np.frombuffer(np.float32(scale0).tobytes(), np.uint32)[0].astype(np.int64)
        bits = (base + np.arange(-(1 << 18), 1 << 18)).astype(np.uint32)
        scales = bits.view(np.float32)
        c = (scales.astype(np.float64) * LOG2E).astype(np.float32)
        mc = (np.float32(smax) * c).astype(np.float32)
        # fma(s, c, -mc): s*c is exact in binary64 (24 x 24 bits) and so is the
        # cancelling difference here, so one rounding to binary32 is the fma.
        x = ((448.0 * a) * c.astype(np.float64) - mc.astype(np.float64)).astype(np.float32)
        hit = np.nonzero(x.view(np.uint32) == np.uint32(target_bits))[0]
        if hit.size:
            return float(scales[hit[0]]), float(a)
    return None


@pytest.mark.parametrize("p_scale", [256.0, 448.0])
@pytest.mark.parametrize("which", [0, 1])
def test_listed_x_values_cast_exactly(p_scale, which):
    import precision_attention_numerics_amd as pan
    target = TARGETS[p_scale][which]
    found = find_scale(target)
    assert found is not None, "no softmax scale reaches the listed x"
    scale, a = found
    N, d = 256, 128
    q = np.zeros((1, 1, N, d), np.float32)
    q[..., 0] = 448.0
    k = np.zeros((1, 1, N, d), np.float32)
    k[..., 0] = 1.0
    k[0, 0, [0, 129], 0] = 448.0           # running max in each block
    k[0, 0, [10, 140], 0] = a              # the key whose x is the listed value
    v = np.random.default_rng(1).standard_normal((1, 1, N, d)).astype(np.float32)
    print(f"S={p_scale} target=0x{target:08x} scale={scale!r} a={a}", flush=True)
    pipe = pan.AttnPipeline(1, 1, 1, N, d)
    gp = pipe.prepare(torch.from_numpy(q).cuda(), torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(),
                      rotate=False, center=False)
    pd = torch.zeros((1, 1, N, N), dtype=torch.uint8, device="cuda")
    kw = dict(p_scale=p_scale, kv_order=1, block_n=128, causal=True, softmax_scale=scale)
    o_dump = pipe.fwd(gp, p_dump=pd, **kw)
    # the timed variant (no dump; block 0 is unmasked for rows 128..255) takes
    # the same fix-up and must give the same output bit for bit
    o_timed = pipe.fwd(gp, **kw)
    torch.cuda.synchronize()
    assert torch.equal(o_dump, o_timed), "timed and dump variants differ"
    op = oracle.prepare(q, k, v)
    assert op.q_desc.ravel()[0] == 1.0 and op.k_desc.ravel()[0] == 1.0
    ref = oracle.attention_fp8(op, p_scale=p_scale, kv_order=1, block_n=128, causal=True, softmax_scale=scale,
                               want_p=True)
    P = pd.cpu().numpy()
    assert p_mismatch(P, ref.p) == 0, np.argwhere(P != ref.p)[:8]
    # the code at the listed x is the correctly rounded one
    x = np.uint32(target).view(np.float32)
    want = oracle.e4m3_encode(np.float32(p_scale) * oracle.exp2_rn32(np.array([x], np.float32)))[0]
    assert P[0, 0, 200, 10] == want and P[0, 0, 200, 140] == want and P[0, 0, 20, 10] == want
