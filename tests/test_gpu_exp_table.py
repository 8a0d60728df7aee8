"""Completeness of the exp2 fix-up table on the GPU: for every P scale the
forward accepts (2^0..2^8 and 448), every binary32 exponent x whose
correctly rounded 2^x lies within a few binary32 steps of an E4M3 rounding
boundary (tests/exp2_candidates.py, pinned on the CPU) is pushed through the
binary32 P-cast kernel, and each P code must equal the code of S * RN32(2^x).
An exponent missing from the table on which the hardware exp2 flips a code
would fail here; away from these candidates a few-ulp exp2 error cannot move
a code.  The FP8 main loop uses the same hardware exp2 and the same table
(only its repair of a listed x differs, covered in test_gpu_exp_fixup.py).

Construction: one KV head, d = 64, key 0 = (0, ..., 0) and key j = (x_j, 0,
..., 0), every query (1, 0, ..., 0), softmax scale RN32(ln 2) so that the
logit factor c = RN32(scale * log2 e) is exactly 1: the scores are x_j
exactly, the running max is 0 from the first block on, and the kernel's
exponent fma(s, c, -m c) is x_j itself."""
import numpy as np
import pytest
import torch

import oracle
import exp2_candidates as ec

pytestmark = pytest.mark.gpu

P_SCALES = [float(2 ** k) for k in range(9)] + [448.0]
CHUNK = 2047
D = 64


def _run(pan, xs: np.ndarray, S: float):
    N = xs.size + 1
    q = np.zeros((1, 1, N, D), np.float32)
    q[..., 0] = 1.0
    k = np.zeros((1, 1, N, D), np.float32)
    k[0, 0, 1:, 0] = xs
    v = np.zeros((1, 1, N, D), np.float32)
    v[0, 0, :, 1] = 1.0
    scale = float(np.float32(np.log(2.0)))
    assert np.float32(np.float64(np.float32(scale)) * 1.4426950408889634) == np.float32(1.0)
    pipe = pan.AttnPipeline(1, 1, 1, N, D)
    dump = torch.zeros((1, 1, N, N), dtype=torch.uint8, device="cuda")
    pipe.fwd_f32(torch.from_numpy(q).cuda(), torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(),
                 p_scale=S, kv_order=0, block_n=128, causal=False, softmax_scale=scale, p_dump=dump)
    torch.cuda.synchronize()
    got = dump[0, 0, 0].cpu().numpy()
    want = np.concatenate([ec.p_codes(np.zeros(1, np.float32), S), ec.p_codes(xs, S)])
    ref = oracle.attention_pcast_f32(q, k, v, softmax_scale=scale, p_scale=S, kv_order=0, block_n=128,
                                     causal=False, rows=np.array([0], np.int32), want_p=True)
    assert np.array_equal(ref.p[0, 0, 0], want), "the oracle's loop disagrees with the candidate codes"
    return got, want


@pytest.mark.parametrize("S", P_SCALES)
def test_every_code_sensitive_exponent(S):
    import precision_attention_numerics_amd as pan
    xs = ec.candidates(S)
    assert xs.size > 500
    bad = []
    for c0 in range(0, xs.size, CHUNK):
        part = xs[c0:c0 + CHUNK]
        got, want = _run(pan, part, S)
        miss = np.nonzero(got != want)[0]
        bad += [hex(int(part[j - 1].view(np.uint32))) for j in miss if j > 0]
        assert got[0] == want[0]
    print(f"[exp table] S={S}: {xs.size} candidate exponents, {len(bad)} code mismatches", flush=True)
    assert not bad, f"exponents whose code differs from S*RN32(2^x): {bad[:10]}"
