"""Shared helpers of the GPU parity tests (not collected by pytest)."""
from __future__ import annotations

import numpy as np
import torch

import oracle


def dev(x: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(x)).cuda()
    return t.to(torch.bfloat16) if dtype == "bf16" else t


def signs_dev(w) -> torch.Tensor:
    return torch.from_numpy(w.signs).cuda()


def compare_prepared(gp, op: oracle.Prepared, N: int, center: bool):
    """Bit-exact comparison of the GPU prologue outputs with the oracle's."""
    q8 = gp.q8.cpu().numpy()
    k8 = gp.k8.cpu().numpy()
    v8t = gp.v8t.cpu().numpy()
    assert np.array_equal(q8[:, :, :N], op.q8), f"Q codes differ at {np.argwhere(q8[:, :, :N] != op.q8)[:5]}"
    assert np.array_equal(k8[:, :, :N], op.k8), f"K codes differ at {np.argwhere(k8[:, :, :N] != op.k8)[:5]}"
    vt = np.swapaxes(v8t, 2, 3)
    assert np.array_equal(vt[:, :, :N], op.v8), f"V codes differ at {np.argwhere(vt[:, :, :N] != op.v8)[:5]}"
    assert not q8[:, :, N:].any() and not k8[:, :, N:].any() and not vt[:, :, N:].any(), "padding not zero"
    assert np.array_equal(gp.q_desc.cpu().numpy(), op.q_desc.ravel())
    assert np.array_equal(gp.k_desc.cpu().numpy(), op.k_desc.ravel())
    assert np.array_equal(gp.v_desc.cpu().numpy(), op.v_desc.ravel())
    if center:
        assert np.array_equal(gp.k_mean.cpu().numpy(), op.k_mean.ravel())
    assert int(gp.status.cpu()[0]) == 0


def max_head_rel(o_gpu: np.ndarray, o_ref: np.ndarray) -> float:
    """Largest per-head relative Frobenius error; a head whose reference is
    exactly zero (an all-zero V head) must be exactly zero too."""
    o64, r64 = np.asarray(o_gpu, np.float64), np.asarray(o_ref, np.float64)
    den = np.sqrt((r64 ** 2).sum(axis=(-2, -1)))
    num = np.sqrt(((o64 - r64) ** 2).sum(axis=(-2, -1)))
    rel = np.where(den > 0, num / np.where(den > 0, den, 1.0), np.where(num > 0, np.inf, 0.0))
    return float(rel.max())


def p_mismatch(p_gpu: np.ndarray, p_ref: np.ndarray) -> int:
    return int((p_gpu != p_ref).sum())
