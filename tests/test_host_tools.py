"""Host-side consistency of the measurement tools: every kernel the HIP
sources define is one the rocprofv3 summary keeps, and the forward kernel that
bench.py names for each mode is the one its committed profile lists."""
import importlib.util
import json
import os
import re

import pytest

from precision_attention_numerics_amd import profile_summary

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "precision_attention_numerics_amd", "csrc")


def _bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_summary_keeps_every_kernel():
    names = set()
    for f in os.listdir(CSRC):
        if f.endswith(".hip"):
            src = open(os.path.join(CSRC, f)).read()
            for m in re.finditer(r"__global__", src):
                head = src[m.end():src.find("{", m.end())]
                names |= set(re.findall(r"\b(k_\w+)\s*\(", head))
    assert names, "no kernels found"
    missing = sorted(n for n in names if not any(k in n for k in profile_summary.KERNELS))
    assert not missing, f"kernels the profile summary would drop: {missing}"


class _Args:
    def __init__(self, tiles, int8):
        self.tile_scales, self.int8_qk = tiles, int8


@pytest.mark.parametrize("tiles,int8,summary", [
    (False, False, "attn_fwd_long_context_32k.json"),
    (True, False, "attn_fwd_tile_scaled_long_context_32k.json"),
    (False, True, "attn_fwd_int8qk_long_context_32k.json"),
])
def test_bench_kernel_name_matches_profile(tiles, int8, summary):
    name = _bench().kernel_name(_Args(tiles, int8))
    rec = json.load(open(os.path.join(ROOT, "profiles", summary)))
    assert name in rec["kernels"], (name, list(rec["kernels"]))
