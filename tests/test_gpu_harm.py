"""Per-head harm of the Hadamard rotation on the Qwen2.5-shaped stacks
(attention-numerics study page, the score definition in "What do these scores
mean?"): for every (layer, head), harm = mean over the texts of
log1p(e_rotated) minus mean over the texts of log1p(e_unrotated), where e is
the head's relative Frobenius error against ideal causal binary64 attention;
a head is harmed iff harm > 0.  Two pairs: rotated against plain, and
centered+rotated against centered (rotation after mean-key centring).

The errors are the GPU's: the forward output of each condition (the
benchmark's launch: S = 256, reverse order, block 128, causal) compared with
the binary64 reference by the library's head-error kernel.  They are checked
against the same metric computed on the host from the same output, and, for
the first and the last layer, the harm from the oracle's emulated outputs must
agree with the GPU's within 1e-3 (the emulated and GPU outputs differ only by
summation order, far below the errors being compared).

The inputs are synthetic (seeded Qwen-like generator), so the harmed-head
counts printed here are this generator's, not the study's."""
import time

import numpy as np
import pytest
import torch

import oracle
import synth
from _gpu_helpers import dev, signs_dev

pytestmark = pytest.mark.gpu
PAIRS = (("rotated", "plain"), ("centered_rotated", "centered"))


def _gpu_errors(pan, w, ref_dev):
    B, hq, N, d = w.q.shape
    hkv = w.k.shape[1]
    pipe = pan.AttnPipeline(B, hq, hkv, N, d)
    q, k, v = dev(w.q, w.dtype), dev(w.k, w.dtype), dev(w.v, w.dtype)
    errs, outs = {}, {}
    for cond, flags in synth.CONDITIONS.items():
        gp = pipe.prepare(q, k, v, signs=signs_dev(w), **flags)
        out = pipe.fwd(gp, p_scale=w.p_scale, kv_order=w.kv_order, block_n=w.block_n, causal=True)
        rel = pipe.head_error(out, ref_dev)
        torch.cuda.synchronize()
        errs[cond] = rel.cpu().numpy().reshape(B, hq)
        outs[cond] = out
    return errs, outs


@pytest.mark.timeout(900)
@pytest.mark.parametrize("model", ["qwen05b", "qwen15b"])
def test_rotation_harm_per_head(model):
    import precision_attention_numerics_amd as pan
    t0 = time.time()
    w = getattr(synth, model)()
    B, hq, N, d = w.q.shape
    layers, texts = w.meta["layers"], w.meta["texts"]
    ideal = oracle.attention_f64(w.q, w.k, w.v, causal=True)
    print(f"[harm] {model}: inputs and binary64 reference in {time.time() - t0:.1f}s", flush=True)
    ref_dev = torch.from_numpy(ideal).cuda()
    errs, outs = _gpu_errors(pan, w, ref_dev)

    # the kernel's metric equals the host's on the same output
    for cond, e in errs.items():
        host = oracle.head_errors(outs[cond].cpu().numpy(), ideal)
        assert np.allclose(e, host, rtol=1e-9, atol=0), cond
        assert np.all(np.isfinite(e)) and np.all(e > 0)

    print(f"[harm] {model} mean log1p(error vs binary64) per condition: "
          + ", ".join(f"{c} {np.log1p(e).mean():.4f}" for c, e in errs.items()), flush=True)

    def harm(rot, unrot, e):
        lr = np.log1p(e[rot]).reshape(layers, texts, hq).mean(axis=1)
        lu = np.log1p(e[unrot]).reshape(layers, texts, hq).mean(axis=1)
        return lr - lu

    summary = {}
    for rot, unrot in PAIRS:
        h = harm(rot, unrot, errs)
        # the oracle's helper gives the same numbers per layer
        for layer in (0, layers - 1):
            sl = slice(layer * texts, (layer + 1) * texts)
            assert np.allclose(h[layer], oracle.harm_scores(errs[rot][sl], errs[unrot][sl]), rtol=0, atol=1e-15)
        summary[(rot, unrot)] = h
        print(f"[harm] {model} {rot} vs {unrot}: harmed {int((h > 0).sum())} of {h.size} heads, "
              f"mean harm {h.mean():+.4f}, median {np.median(h):+.4f}, min {h.min():+.4f}, max {h.max():+.4f}",
              flush=True)

    # cross-check against the emulator on the first and the last layer
    for layer in (0, layers - 1):
        sl = slice(layer * texts, (layer + 1) * texts)
        emu = {}
        for cond, flags in synth.CONDITIONS.items():
            op = oracle.prepare(w.q[sl], w.k[sl], w.v[sl], signs=w.signs, **flags)
            r = oracle.attention_fp8(op, p_scale=w.p_scale, kv_order=w.kv_order, block_n=w.block_n, causal=True)
            emu[cond] = oracle.head_errors(r.out, ideal[sl])
        for rot, unrot in PAIRS:
            he = oracle.harm_scores(emu[rot], emu[unrot])
            hg = summary[(rot, unrot)][layer]
            assert np.max(np.abs(he - hg)) <= 1e-3, (layer, rot, np.max(np.abs(he - hg)))
        print(f"[harm] {model} layer {layer}: emulator harm agrees", flush=True)
    print(f"[harm] {model}: done in {time.time() - t0:.1f}s", flush=True)
