"""Throughput of the causal FP8 attention forward on one MI355X.

Workload: batch 1, 32 query heads, 8 KV heads (GQA 4:1), head_dim 128,
N = 32768 tokens, causal, BF16 operands from the sink generator (Delta = 8,
4-token sink block), FP8 E4M3 for Q.K^T and P.V, P scale S = 256, reverse KV
order, KV block 128; conditions "centered_rotated" (the timed step) and
"rotated" (reported beside it).

One step = the whole hot path on resident inputs: fp8_attn_prepare (mean key,
Hadamard, scales, E4M3 codes) + fp8_attn_fwd (online-softmax FP8 attention)
+ fp8_attn_head_error (per-head relative Frobenius error against the
binary64 reference rows).  value = algorithmic FLOP of the causal forward
(4*B*Hq*N^2*d/2) per step time.  `detail` also carries the forward time of
the Qwen2.5-0.5B and -1.5B shaped stacks (N = 1024, all layers x 3 texts in
one launch).

The CPU oracle (bit-faithful emulator and binary64 reference) runs on a
bounded sample of query rows as the cpu_baseline leg; its reference rows feed
the per-head error and its emulated rows check the GPU output.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

FP8_DENSE_PEAK_TFLOPS = 5000.0   # MI355X dense FP8 matrix peak
HBM_PEAK_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--seqlen", type=int, default=32768)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-qwen", action="store_true", help="skip the Qwen-shaped stacks' forward timing in detail")
    ap.add_argument("--qwen-only", action="store_true",
                    help="only time the Qwen-shaped stacks' forward (one JSON line of their detail; for profiling)")
    ap.add_argument("--tile-scales", action="store_true",
                    help="one Q/K scale per 128-token tile (the variant) instead of per (batch, head)")
    ap.add_argument("--int8-qk", action="store_true",
                    help="Q/K as int8 codes with exact integer scores (the INT8-QK / FP8-PV variant)")
    ap.add_argument("--sample-tiles", type=int, default=3, help="query tiles per head in the CPU sample")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="only run a plain device copy (read + write of this many MiB), for scaling HBM counters")
    return ap.parse_args()


def copy_calibration(mib: int, steps: int):
    """A plain elementwise copy kernel of known size: reads and writes mib MiB."""
    import torch
    n = mib * (1 << 20) // 4
    x = torch.randn(n, device="cuda")
    y = torch.empty_like(x)
    for _ in range(steps):
        torch.mul(x, 1.0, out=y)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": n * 4, "copy_calibration_bytes_written": n * 4, "launches": steps}))


def profiled_traffic(kernel: str, summary: str = "attn_fwd_long_context_32k.json"):
    """HBM bytes per launch of the forward kernel from the committed rocprofv3
    counters (FETCH_SIZE + WRITE_SIZE, copy-scaled) in profiles/<summary>, or
    None when the kernel sources have changed since they were taken."""
    from precision_attention_numerics_amd.profile_summary import kernel_source_sha256
    path = os.path.join(ROOT, "profiles", summary)
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("kernel_source_sha256") != kernel_source_sha256():
        return None
    for name, v in rec["kernels"].items():
        if name.startswith(kernel):
            return v.get("read_bytes", 0.0) + v.get("write_bytes", 0.0)
    return None


def provenance(torch, pan) -> dict:
    """What the line was measured on: the device, and the build of the
    library that ran (the hash of the sources it was built from)."""
    props = torch.cuda.get_device_properties(0)
    return {"device": torch.cuda.get_device_name(0), "arch": getattr(props, "gcnArchName", ""),
            "compute_units": props.multi_processor_count, "library_build": pan._abi.build_info(),
            "torch": torch.__version__, "hip": torch.version.hip}


def kernel_name(args) -> str:
    """The forward kernel the timed launch runs (as rocprofv3 names it)."""
    return "k_attn_fwd_pipe<true, true, %s, 2, %s>" % ("true" if args.tile_scales else "false",
                                                       "true" if args.int8_qk else "false")


def sample_rows(N: int, tiles: int) -> np.ndarray:
    """First, middle and last 128-row query tiles (evenly spaced tiles when
    more are asked for)."""
    nt = (N + 127) // 128
    idx = np.unique(np.linspace(0, nt - 1, tiles).round().astype(int))
    rows = np.concatenate([np.arange(t * 128, min(N, t * 128 + 128)) for t in idx])
    return rows.astype(np.int32)


def qwen_stacks(pan, synth, torch, args) -> dict:
    """Forward of the Qwen2.5-0.5B and -1.5B shaped stacks (all layers x 3 texts
    as one batch, N = 1024, centred and rotated, S = 256, reverse, block 128):
    mean HIP-event time of the forward launch on the current stream."""
    out = {}
    for name, gen in (("qwen2.5-0.5b_stack", synth.qwen05b), ("qwen2.5-1.5b_stack", synth.qwen15b)):
        t0 = time.time()
        w = gen()
        B, hq, N, d = w.q.shape
        hkv = w.k.shape[1]
        pipe = pan.AttnPipeline(B, hq, hkv, N, d)
        q = torch.from_numpy(w.q).cuda().to(torch.bfloat16)
        k = torch.from_numpy(w.k).cuda().to(torch.bfloat16)
        v = torch.from_numpy(w.v).cuda().to(torch.bfloat16)
        signs = torch.from_numpy(w.signs).cuda()
        prep = pipe.prepare(q, k, v, rotate=True, center=True, signs=signs)
        o = torch.empty((B, hq, N, d), dtype=torch.float32, device="cuda")
        for _ in range(args.warmup):
            pipe.fwd(prep, p_scale=256.0, kv_order=1, block_n=128, causal=True, out=o)
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
        for a, b in evs:
            a.record()
            pipe.fwd(prep, p_scale=256.0, kv_order=1, block_n=128, causal=True, out=o)
            b.record()
        torch.cuda.synchronize()
        ms = float(np.mean([a.elapsed_time(b) for a, b in evs]))
        flop = 4.0 * B * hq * N * N * d / 2.0
        tf = flop / (ms * 1e-3) / 1e12
        out[name] = {"shape": f"B={B} (layers x 3 texts) Hq={hq} Hkv={hkv} N={N} d={d}", "fwd_ms": ms,
                     "fwd_tflops": tf, "fwd_frac_of_fp8_peak": tf / FP8_DENSE_PEAK_TFLOPS}
        print(f"[bench] {name}: {out[name]} (inputs {time.time() - t0:.1f}s)", file=sys.stderr, flush=True)
        del q, k, v, prep, o
        torch.cuda.empty_cache()
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the library has no multi-GPU path. "
              "Sharding by head would need no communication between GPUs.", file=sys.stderr)
        sys.exit(2)
    import torch

    if args.copy_calibration_mib:
        copy_calibration(args.copy_calibration_mib, args.steps)
        return

    import precision_attention_numerics_amd as pan
    import synth

    assert torch.cuda.is_available(), "bench.py needs the GPU"
    torch.cuda.set_device(0)
    if args.qwen_only:
        print(json.dumps({"detail": qwen_stacks(pan, synth, torch, args)}), flush=True)
        return
    t0 = time.time()
    w = synth.long_context(N=args.seqlen)
    B, hq, N, d = w.q.shape
    hkv = w.k.shape[1]
    print(f"[bench] inputs generated in {time.time() - t0:.1f}s: B={B} hq={hq} hkv={hkv} N={N} d={d}", file=sys.stderr, flush=True)
    q = torch.from_numpy(w.q).cuda().to(torch.bfloat16)
    k = torch.from_numpy(w.k).cuda().to(torch.bfloat16)
    v = torch.from_numpy(w.v).cuda().to(torch.bfloat16)
    signs = torch.from_numpy(w.signs).cuda()
    pipe = pan.AttnPipeline(B, hq, hkv, N, d)
    rows = sample_rows(N, args.sample_tiles)
    rows_dev = torch.from_numpy(rows).cuda()
    flop = 4.0 * B * hq * N * N * d / 2.0

    # ---- CPU oracle leg: bounded sample, gives the binary64 reference rows
    cpu = None
    ref_rows = {}
    emu_rows = {}
    if not args.no_cpu_baseline:
        import oracle
        threads = oracle._threads(None)
        pairs = float(B * hq * np.sum(rows + 1))                      # visible (query, key) pairs of the sample
        t_loop = t_prep = 0.0
        for cond in ("centered_rotated", "rotated"):
            fl = synth.CONDITIONS[cond]
            ta = time.perf_counter()
            op = oracle.prepare(w.q, w.k, w.v, signs=w.signs, tiles=args.tile_scales, int8=args.int8_qk, **fl)
            tm = time.perf_counter()
            emu = oracle.attention_fp8(op, p_scale=256.0, kv_order=1, block_n=128, causal=True, rows=rows)
            tb = time.perf_counter()
            if cond == "centered_rotated":
                t_prep, t_loop = tm - ta, tb - tm
            emu_rows[cond] = emu.out
            print(f"[bench] oracle emulator {cond}: prologue {tm - ta:.1f}s, main loop {tb - tm:.1f}s",
                  file=sys.stderr, flush=True)
        ta = time.perf_counter()
        ideal = oracle.attention_f64(w.q, w.k, w.v, causal=True, rows=rows)
        t_ideal = time.perf_counter() - ta
        ref_rows["f64"] = ideal
        print(f"[bench] oracle binary64 reference: {t_ideal:.1f}s", file=sys.stderr, flush=True)
        cpu = {"value": 4.0 * d * pairs / t_loop / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
               "sample": (f"bit-faithful emulator main loop on {rows.size} query rows x {hq} heads (first/middle/last "
                          f"128-row tiles: {pairs:.3g} visible query-key pairs), centered_rotated: {t_loop:.1f}s; "
                          f"value = 4*d FLOP per pair over that time.  Not in value: the emulated prologue on all "
                          f"{N} tokens ({t_prep:.1f}s) and the binary64 reference on the same rows ({t_ideal:.1f}s)")}

    ref = torch.from_numpy(ref_rows["f64"]).cuda() if ref_rows else torch.zeros((B, hq, rows.size, d), dtype=torch.float64, device="cuda")
    prep = pipe.alloc_prepared(args.tile_scales, args.int8_qk)
    out = torch.empty((B, hq, N, d), dtype=torch.float32, device="cuda")
    rel = torch.empty(B * hq, dtype=torch.float64, device="cuda")

    def step(cond, ev=None):
        fl = synth.CONDITIONS[cond]
        if ev is not None:
            ev[0].record()
        pipe.prepare(q, k, v, signs=signs, prep=prep, tiles=args.tile_scales, int8=args.int8_qk, **fl)
        if ev is not None:
            ev[1].record()
        pipe.fwd(prep, p_scale=256.0, kv_order=1, block_n=128, causal=True, out=out)
        if ev is not None:
            ev[2].record()
        pipe.head_error(out, ref, rows=rows_dev, rel_err=rel)
        if ev is not None:
            ev[3].record()

    results = {}
    for cond in ("rotated", "centered_rotated"):
        for _ in range(args.warmup):
            step(cond)
        torch.cuda.synchronize()
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
        torch.cuda.synchronize()
        ta = time.perf_counter()
        for i in range(args.steps):
            step(cond, evs[i])
        torch.cuda.synchronize()
        tb = time.perf_counter()
        prep_ms = np.mean([e[0].elapsed_time(e[1]) for e in evs])
        fwd_all = [e[1].elapsed_time(e[2]) for e in evs]
        fwd_ms = np.mean(fwd_all)
        err_ms = np.mean([e[2].elapsed_time(e[3]) for e in evs])
        o_rows = out[:, :, rows_dev.long()].cpu().numpy()
        rel_np = rel.cpu().numpy()
        # prologue bytes: minimal = BF16 Q/K/V read once + one code byte
        # written per element; two-pass = the max pass and the quantise pass
        # each read Q/K/V (plus one more read of K for the mean when centred)
        elems = B * (hq + 2 * hkv) * N * d
        min_bytes = 3 * elems
        two_pass = 5 * elems + (2 * B * hkv * N * d if synth.CONDITIONS[cond]["center"] else 0)
        res = {"ms_per_step": (tb - ta) * 1e3 / args.steps, "prepare_ms": float(prep_ms), "fwd_ms": float(fwd_ms),
               "fwd_median_ms": float(np.median(fwd_all)), "head_error_ms": float(err_ms),
               "prepare_GBps_minimal_bytes": min_bytes / (prep_ms * 1e-3) / 1e9,
               "prepare_GBps_two_pass_bytes": two_pass / (prep_ms * 1e-3) / 1e9}
        if ref_rows:
            lg = np.log1p(rel_np)
            res["log1p_rel_err_vs_f64"] = {"mean": float(lg.mean()), "max": float(lg.max()), "min": float(lg.min())}
            import oracle
            res["max_head_rel_err_vs_emulator"] = float(oracle.head_errors(o_rows, emu_rows[cond]).max())
        results[cond] = res
        print(f"[bench] {cond}: {res}", file=sys.stderr, flush=True)

    if not args.no_qwen:
        results.update(qwen_stacks(pan, synth, torch, args))

    main_res = results["centered_rotated"]
    fwd_tflops = flop / (main_res["fwd_ms"] * 1e-3) / 1e12
    value = flop / (main_res["ms_per_step"] * 1e-3) / 1e12
    line = {
        "metric": "causal FP8 attn fwd TFLOP/s (% of FP8 MFMA peak) + per-head rel-Frobenius err",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(main_res["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8 (Q.K) + e4m3 (P.V)" if args.int8_qk else "e4m3",
        "data": "synthetic",
        "config": {"workload": "long-context causal FP8 attention forward, B=1, Hq=32, Hkv=8, d=128, N=%d, "
                               "BF16 sink-generator operands (Delta=8, 4 sinks), S=256, reverse KV order, block 128" % N,
                   "condition": "centered_rotated",
                   "qk_scales": "per 128-token tile" if args.tile_scales else "per (batch, head)",
                   "qk_codes": "int8" if args.int8_qk else "e4m3",
                   "pct_of_fp8_peak": round(100 * value / FP8_DENSE_PEAK_TFLOPS, 2)},
        "roofline": {"bound": "mfma", "achieved": round(fwd_tflops, 2), "peak": FP8_DENSE_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(fwd_tflops / FP8_DENSE_PEAK_TFLOPS, 4),
                     "traffic": profiled_traffic(kernel_name(args),
                         ("attn_fwd_tile_scaled_long_context_32k.json" if args.tile_scales else
                          "attn_fwd_int8qk_long_context_32k.json" if args.int8_qk else
                          "attn_fwd_long_context_32k.json")),
                     "kernel": kernel_name(args),
                     "flop_per_launch": flop},
        "cpu_baseline": cpu,
        "detail": results,
        "provenance": provenance(torch, pan),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
