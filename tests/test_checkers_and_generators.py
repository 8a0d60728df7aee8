"""The parity checkers and the seeded generators themselves, on the CPU.

Checkers: the comparisons the GPU tests rely on must fail on a planted fault.
A prologue laid out as the GPU writes it (codes padded to whole 128-token
tiles, V transposed), built here from the oracle's own output, passes
compare_prepared; one flipped code byte, one changed descale bit, nonzero
padding or a set status word each fail it.  An output off by 3e-3 in one
head's relative Frobenius norm exceeds the 2e-3 bar of max_head_rel, and a
nonzero output where the reference head is exactly zero is infinitely wrong.
p_mismatch counts one changed P~ code as one.

Generators: every workload is a pure function of its seed (same seed, same
bytes; another seed, other values), so that the oracle and the kernels see the
same inputs in every run."""
import types

import numpy as np
import pytest
import torch

import oracle
import synth
from _gpu_helpers import compare_prepared, max_head_rel, p_mismatch


def _gpu_layout(op: oracle.Prepared, N: int, center: bool):
    """The oracle's prologue in the device layout of fp8_attn_prepare."""
    B, hq, _, d = op.q8.shape
    hkv = op.k8.shape[1]
    Np = (N + 127) // 128 * 128
    q8 = np.zeros((B, hq, Np, d), np.uint8)
    k8 = np.zeros((B, hkv, Np, d), np.uint8)
    v8t = np.zeros((B, hkv, d, Np), np.uint8)
    q8[:, :, :N] = op.q8
    k8[:, :, :N] = op.k8
    v8t[:, :, :, :N] = np.swapaxes(op.v8, 2, 3)
    t = torch.from_numpy
    return types.SimpleNamespace(
        q8=t(q8), k8=t(k8), v8t=t(v8t), q_desc=t(op.q_desc.ravel().copy()), k_desc=t(op.k_desc.ravel().copy()),
        v_desc=t(op.v_desc.ravel().copy()),
        k_mean=t(op.k_mean.ravel().copy()) if center else None, status=torch.zeros(1, dtype=torch.int32))


@pytest.fixture(scope="module")
def prepared():
    w = synth.qwen_like(1, 4, 2, 64, seed=910, N=200, texts=1)
    op = oracle.prepare(w.q, w.k, w.v, rotate=True, center=True, signs=w.signs)
    return op, 200


def test_compare_prepared_accepts_the_oracles_own_prologue(prepared):
    op, N = prepared
    compare_prepared(_gpu_layout(op, N, True), op, N, center=True)


@pytest.mark.parametrize("fault", ["q_code", "k_code", "v_code", "q_desc", "v_desc", "k_mean", "padding",
                                   "status"])
def test_compare_prepared_rejects_each_planted_fault(prepared, fault):
    op, N = prepared
    gp = _gpu_layout(op, N, True)
    if fault == "q_code":
        gp.q8[0, 1, 57, 3] ^= 0x01
    elif fault == "k_code":
        gp.k8[0, 1, N - 1, 63] ^= 0x80
    elif fault == "v_code":
        gp.v8t[0, 0, 5, 0] ^= 0x10
    elif fault == "q_desc":
        gp.q_desc.view(torch.int32)[2] ^= 1
    elif fault == "v_desc":
        gp.v_desc.view(torch.int32)[1] ^= 1
    elif fault == "k_mean":
        gp.k_mean.view(torch.int32)[7] ^= 1
    elif fault == "padding":
        gp.k8[0, 0, N, 0] = 1
    else:
        gp.status[0] = 1
    with pytest.raises(AssertionError):
        compare_prepared(gp, op, N, center=True)


def test_max_head_rel_catches_a_3e_3_error_in_one_head():
    g = np.random.default_rng(3)
    ref = g.standard_normal((2, 3, 50, 16))
    assert max_head_rel(ref, ref) == 0.0
    out = ref.copy()
    out[1, 2] += 3e-3 * np.linalg.norm(ref[1, 2]) * g.standard_normal((50, 16)) / np.sqrt(50 * 16)
    err = max_head_rel(out, ref)
    assert err > 2e-3, err
    assert abs(err - 3e-3) < 5e-4, err
    zero_ref = ref.copy()
    zero_ref[0, 0] = 0.0
    assert max_head_rel(zero_ref, zero_ref) == 0.0
    bad = zero_ref.copy()
    bad[0, 0, 0, 0] = 1e-30
    assert max_head_rel(bad, zero_ref) == np.inf


def test_p_mismatch_counts_each_changed_code():
    p = np.random.default_rng(4).integers(0, 127, (2, 8, 8), dtype=np.uint8)
    q = p.copy()
    assert p_mismatch(q, p) == 0
    q[1, 3, 5] ^= 0x01
    assert p_mismatch(q, p) == 1


GENERATORS = {
    "illustration": lambda s: synth.illustration(seed=s, N=64),
    "pcast_sweep": lambda s: synth.pcast_sweep(6.0, seed=s, N=256),
    "qwen_like": lambda s: synth.qwen_like(2, 6, 2, 64, seed=s, N=96, texts=2),
    "long_context": lambda s: synth.long_context(seed=s, N=256, hq=4, hkv=2),
}


@pytest.mark.parametrize("name", sorted(GENERATORS))
def test_generators_are_functions_of_their_seed(name):
    gen = GENERATORS[name]
    a, b, c = gen(11), gen(11), gen(12)
    for field in ("q", "k", "v"):
        x, y, z = getattr(a, field), getattr(b, field), getattr(c, field)
        assert x.dtype == y.dtype and x.shape == y.shape
        assert np.array_equal(x.view(np.uint8), y.view(np.uint8)), f"{name}.{field} differs for one seed"
        assert not np.array_equal(x, z), f"{name}.{field} does not depend on the seed"
    assert np.array_equal(synth.rotation_signs(128), synth.rotation_signs(128))
