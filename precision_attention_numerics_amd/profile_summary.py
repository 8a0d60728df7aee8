"""Summarise rocprofv3 CSV output of bench.py runs into a short text table.

usage: python -m precision_attention_numerics_amd.profile_summary PROFDIR > summary.md
       python -m precision_attention_numerics_amd.profile_summary PROFDIR --json OUT.json
(the JSON records the forward kernel's scaled HBM bytes per launch and the
sha256 of the kernel source they were measured on)

PROFDIR holds the sub-directories written by these commands (run from /tmp,
TMPDIR=/tmp, R = repository root):
  trace: rocprofv3 --kernel-trace --stats -S --output-format csv -d PROFDIR/trace -o trace -- python3 R/bench.py --no-cpu-baseline --no-qwen --steps 20 --warmup 5
  fetch: rocprofv3 --pmc FETCH_SIZE --output-format csv -d PROFDIR/fetch -o fetch -- python3 R/bench.py --no-cpu-baseline --no-qwen --steps 2 --warmup 0
  write: rocprofv3 --pmc WRITE_SIZE --output-format csv -d PROFDIR/write -o write -- python3 R/bench.py --no-cpu-baseline --no-qwen --steps 2 --warmup 0
  sq:    rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CYCLES SQ_INSTS_VALU SQ_INSTS_MFMA SQ_INSTS_VALU_TRANS_F32 SQ_INSTS_LDS SQ_LDS_BANK_CONFLICT SQ_VALU_MFMA_COEXEC_CYCLES GRBM_GUI_ACTIVE --output-format csv -d PROFDIR/sq -o sq -- python3 R/bench.py --no-cpu-baseline --no-qwen --steps 2 --warmup 0
  copyf: rocprofv3 --pmc FETCH_SIZE --output-format csv -d PROFDIR/copyf -o copyf -- python3 R/bench.py --copy-calibration-mib 1024 --steps 3
  copyw: rocprofv3 --pmc WRITE_SIZE --output-format csv -d PROFDIR/copyw -o copyw -- python3 R/bench.py --copy-calibration-mib 1024 --steps 3
"""
from __future__ import annotations

import collections
import csv
import os
import sys

KERNELS = ("k_attn_fwd", "k_attn_pcast", "k_amax", "k_prefix_max", "k_quant_qk", "k_quant_vt",
           "k_kmean_partial", "k_kmean_final", "k_head_err_partial", "k_head_err_final", "k_fill2_u32")
COPY_BYTES = 1024 * (1 << 20)


def short(name: str) -> str:
    name = name.replace("void ", "").replace("fp8a::", "").replace("(anonymous namespace)::", "")
    return name.split("(")[0]


def counters(path: str):
    """Mean counter value per (kernel, counter) over dispatches."""
    agg = collections.defaultdict(list)
    for r in csv.DictReader(open(path)):
        agg[(short(r["Kernel_Name"]), r["Counter_Name"])].append(float(r["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in agg.items()}


def dispatch_median_us(d: str) -> dict:
    """Median duration per kernel over its dispatches (the average includes the
    first launches, which run while the clocks ramp up)."""
    per = collections.defaultdict(list)
    for r in csv.DictReader(open(os.path.join(d, "trace", "trace_kernel_trace.csv"))):
        per[short(r["Kernel_Name"])].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    out = {}
    for k, v in per.items():
        v = sorted(v)
        out[k] = v[len(v) // 2] if len(v) % 2 else 0.5 * (v[len(v) // 2 - 1] + v[len(v) // 2])
    return out


def main(d: str):
    stats = list(csv.DictReader(open(os.path.join(d, "trace", "trace_kernel_stats.csv"))))
    med = dispatch_median_us(d)
    fetch = counters(os.path.join(d, "fetch", "fetch_counter_collection.csv"))
    write = counters(os.path.join(d, "write", "write_counter_collection.csv"))
    sq = counters(os.path.join(d, "sq", "sq_counter_collection.csv"))
    copyf = counters(os.path.join(d, "copyf", "copyf_counter_collection.csv"))
    copyw = counters(os.path.join(d, "copyw", "copyw_counter_collection.csv"))
    cf = [v for (k, c), v in copyf.items() if c == "FETCH_SIZE" and "elementwise" in k]
    cw = [v for (k, c), v in copyw.items() if c == "WRITE_SIZE" and "elementwise" in k]
    f_scale = COPY_BYTES / (max(cf) * 1024) if cf else float("nan")
    w_scale = COPY_BYTES / (max(cw) * 1024) if cw else float("nan")
    print("| kernel | calls | avg us | median us | HBM read MB/launch | HBM write MB/launch |")
    print("|---|---|---|---|---|---|")
    for r in stats:
        k = short(r["Name"])
        if not any(x in k for x in KERNELS):
            continue
        fs = fetch.get((k, "FETCH_SIZE"))
        ws = write.get((k, "WRITE_SIZE"))
        rd = f"{fs * 1024 * f_scale / 1e6:.1f}" if fs is not None else "-"
        wr = f"{ws * 1024 * w_scale / 1e6:.1f}" if ws is not None else "-"
        print(f"| {k} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | {med.get(k, float('nan')):.1f} | {rd} | {wr} |")
    print(f"\ncounter scale from the plain 1 GiB copy: FETCH_SIZE x{f_scale:.3f}, WRITE_SIZE x{w_scale:.3f}\n")
    att = [k for (k, c) in sq if "k_attn_fwd" in k]
    for k in sorted(set(att)):
        g = {c: v for (kk, c), v in sq.items() if kk == k}
        act = g.get("GRBM_GUI_ACTIVE", float("nan"))
        simds = 256 * 4
        print(f"SQ counters, {k} (per launch):")
        for c in sorted(g):
            print(f"  {c}: {g[c]:.4g}")
        if act == act:
            # GRBM_GUI_ACTIVE is summed over the 8 XCDs: cycles per XCD = act / 8
            cyc = act / 8
            print(f"  MFMA busy fraction per SIMD: {g.get('SQ_VALU_MFMA_BUSY_CYCLES', 0) / simds / cyc:.3f}")
            print(f"  MFMA/VALU co-issue fraction: {g.get('SQ_VALU_MFMA_COEXEC_CYCLES', 0) / simds / cyc:.3f}")
            print(f"  VALU instructions per MFMA: {g.get('SQ_INSTS_VALU', 0) / max(g.get('SQ_INSTS_MFMA', 1), 1):.2f}")
            m_us = med.get(k)
            if m_us:
                # busy cycles per XCD over the same kernel's median duration in
                # the trace run: the engine clock it ran at, and the dense FP8
                # peak at that clock (256 CUs x 8192 FLOP per clock)
                ghz = cyc / (m_us * 1e3)
                print(f"  engine clock estimate (GRBM_GUI_ACTIVE / 8 / trace median): {ghz:.2f} GHz; "
                      f"dense FP8 peak at that clock: {256 * 8192 * ghz / 1e3:.0f} TFLOP/s")


# every source the forward kernels are compiled from: counters recorded for
# one version of the code are not used for another (comments and layout do
# not count: they are removed before hashing)
KERNEL_SOURCES = ("attn_fwd.hip", "attn_fwd32.hip", "attn_common.hpp", "attn.hpp", "device_common.hpp")


def _code_only(text: str) -> str:
    import re
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_source_sha256() -> str:
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc")
    for name in KERNEL_SOURCES:
        h.update(name.encode())
        h.update(_code_only(open(os.path.join(csrc, name)).read()).encode())
    return h.hexdigest()


def write_json(d: str, out: str):
    import json
    fetch = counters(os.path.join(d, "fetch", "fetch_counter_collection.csv"))
    write = counters(os.path.join(d, "write", "write_counter_collection.csv"))
    copyf = counters(os.path.join(d, "copyf", "copyf_counter_collection.csv"))
    copyw = counters(os.path.join(d, "copyw", "copyw_counter_collection.csv"))
    f_scale = COPY_BYTES / (max(v for (k, c), v in copyf.items() if "elementwise" in k) * 1024)
    w_scale = COPY_BYTES / (max(v for (k, c), v in copyw.items() if "elementwise" in k) * 1024)
    res = {"kernel_source_sha256": kernel_source_sha256(), "kernels": {}}
    for (k, c), v in fetch.items():
        if "k_attn_fwd" in k:
            res["kernels"].setdefault(k, {})["read_bytes"] = v * 1024 * f_scale
    for (k, c), v in write.items():
        if "k_attn_fwd" in k:
            res["kernels"].setdefault(k, {})["write_bytes"] = v * 1024 * w_scale
    res["fetch_scale"], res["write_scale"] = f_scale, w_scale
    json.dump(res, open(out, "w"), indent=1)


if __name__ == "__main__":
    if "--json" in sys.argv:
        write_json(sys.argv[1], sys.argv[sys.argv.index("--json") + 1])
    else:
        main(sys.argv[1])
