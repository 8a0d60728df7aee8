"""The C-ABI library on the host: it loads, exports every function
include/fp8_attn.h declares, and its host-side validation rejects bad
arguments before any launch (no GPU is touched: every call below fails a check
that precedes the first HIP call)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "precision_attention_numerics_amd", "libfp8attn.so")
HEADER = os.path.join(ROOT, "include", "fp8_attn.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.fail("libfp8attn.so is not built: run __graft_entry__.build()")
    return ctypes.CDLL(LIB)


@pytest.fixture(scope="module")
def abi():
    import precision_attention_numerics_amd._abi as abi
    return abi


def declared():
    return sorted(set(re.findall(r"\b(fp8_attn_\w+)\s*\(", open(HEADER).read())))


def test_header_declares_the_boundary():
    names = declared()
    for must in ("fp8_attn_prepare", "fp8_attn_fwd", "fp8_attn_head_error", "fp8_attn_strerror"):
        assert must in names


def test_every_declared_symbol_exported(lib):
    for name in declared():
        assert hasattr(lib, name), name


def test_no_torch_types_in_header():
    text = open(HEADER).read()
    assert "torch" not in text.lower().replace("torch types", "") and "at::" not in text


def test_pure_host_helpers(abi):
    assert abi.padded_seqlen(1) == 128 and abi.padded_seqlen(128) == 128 and abi.padded_seqlen(129) == 256
    assert abi.padded_seqlen(0) == 0
    assert abi.padded_seqlen(1 << 30) == 1 << 30 and abi.padded_seqlen((1 << 30) + 1) == 0
    assert abi.padded_seqlen(2**31 - 1) == 0
    for st in range(-6, 1):
        assert abi.strerror(st) != "unknown status"
    assert abi.strerror(-99) == "unknown status"


def test_workspace_sizes(abi):
    s = abi.make_shape(1, 32, 8, 32768, 128)
    base = abi.prepare_workspace_bytes(s, 0)
    cen = abi.prepare_workspace_bytes(s, abi.FP8A_CENTER_K)
    assert base >= (32 + 16) * 4 and cen > base
    assert cen - base >= 8 * 512 * 128 * 8          # 512 chunk partials per KV head and channel
    assert abi.head_error_workspace_bytes(s, 32768) >= 32 * 2 * 8
    tiles = abi.prepare_workspace_bytes(s, abi.FP8A_TILE_SCALES)
    assert tiles - base >= (32 + 8) * (256 - 1) * 4      # one max slot per 128-token tile of Q and K heads
    bad = abi.make_shape(1, 3, 2, 16, 128)           # hq % hkv != 0
    assert abi.prepare_workspace_bytes(bad, 0) == 0


FAKE = ctypes.c_void_p(1 << 20)   # aligned, never dereferenced: every call fails validation first


def _no_gpu():
    """The fake-pointer calls are only made where no GPU is visible, so that a
    validation bug could never turn into a launch on real hardware."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("fake-pointer validation tests run on hosts without a GPU")


def _prep(abi, shape, dtype=1, flags=0, signs=FAKE, ws=FAKE, ws_bytes=1 << 30, q=FAKE):
    return abi._lib.fp8_attn_prepare(ctypes.byref(shape), dtype, q, FAKE, FAKE, flags, signs, FAKE, FAKE, FAKE,
                                     FAKE, FAKE, FAKE, None, None, ws, ws_bytes, None)


def _fwd(abi, shape, **kw):
    a = dict(dtype=3, scale=0.088, S=256.0, order=1, bn=128, causal=1, out=FAKE, k_sink=0, desc=FAKE)
    a.update(kw)
    return abi._lib.fp8_attn_fwd(ctypes.byref(shape), a["dtype"], FAKE, FAKE, FAKE, a["desc"], a["desc"], a["desc"],
                                 a["scale"], a["S"], a["order"], a["bn"], a["causal"], a["out"], None, None, None,
                                 None, a["k_sink"], None)


def test_prepare_rejects(abi):
    _no_gpu()
    ok = abi.make_shape(1, 2, 1, 64, 64)
    assert _prep(abi, abi.make_shape(1, 2, 1, 64, 96)) == -2          # head_dim
    assert _prep(abi, abi.make_shape(1, 3, 2, 64, 64)) == -2          # GQA ratio
    assert _prep(abi, abi.make_shape(0, 2, 1, 64, 64)) == -2          # batch
    assert _prep(abi, abi.make_shape(1, 2, 1, 0, 64)) == -2           # seqlen
    assert _prep(abi, abi.make_shape(1, 2, 1, (1 << 30) + 1, 64)) == -2   # seqlen above 2^30
    assert _prep(abi, abi.make_shape(32768, 2, 1, 64, 64)) == -2      # batch * hq above the grid limit
    assert _prep(abi, abi.make_shape(21845, 3, 3, 64, 64)) == -2      # batch * (hq + 2 hkv) above it
    assert _prep(abi, abi.make_shape(7281, 3, 3, 64, 64), ws_bytes=1) == -5   # 65529 heads in all: accepted
    assert _prep(abi, abi.make_shape(4096, 8, 1, 1 << 30, 64)) == -2  # forward grid beyond 31 bits
    assert _prep(abi, ok, dtype=2) == -3                               # f64 input
    assert _prep(abi, ok, flags=32) == -4                              # unknown flag
    assert _prep(abi, ok, flags=abi.FP8A_TILE_SCALES, ws_bytes=1) == -5   # tile maxima need workspace too
    assert _prep(abi, ok, flags=abi.FP8A_PREFIX_SCALES) == -4                # prefix scales need tiles
    # a centred prefix prologue is accepted (it then fails only on the missing workspace)
    assert _prep(abi, ok, flags=abi.FP8A_PREFIX_SCALES | abi.FP8A_TILE_SCALES | abi.FP8A_CENTER_K, ws_bytes=1) == -5
    assert _prep(abi, ok, flags=abi.FP8A_INT8_QK | abi.FP8A_TILE_SCALES) == -3         # int8 only per head
    assert _prep(abi, ok, q=None) == -1
    assert _prep(abi, ok, flags=abi.FP8A_ROTATE_QK, signs=None) == -1
    assert _prep(abi, ok, ws=None) == -5
    assert _prep(abi, ok, ws_bytes=1) == -5
    assert _prep(abi, ok, q=ctypes.c_void_p((1 << 20) + 8)) == -2     # misaligned
    st = abi.make_shape(1, 2, 1, 64, 64)
    st.q_stride[:] = [8192, 4096, 63]                                  # row stride not a multiple of 8
    assert _prep(abi, st) == -2
    assert abi._lib.fp8_attn_prepare(None, 1, FAKE, FAKE, FAKE, 0, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                     None, None, FAKE, 1 << 30, None) == -1


def test_prepare_noalloc_rejects(abi):
    """The no-alloc prologue validates like fp8_attn_prepare and refuses a
    shape whose workspace exceeds its fixed scratch, before any HIP call."""
    _no_gpu()
    f = abi._lib.fp8_attn_prepare_noalloc

    def call(shape, flags=0, q=FAKE, signs=FAKE):
        return f(ctypes.byref(shape), 1, q, FAKE, FAKE, flags, signs, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None,
                 None, None)
    big = abi.make_shape(1, 32, 8, 65536, 128)
    cen = abi.FP8A_ROTATE_QK | abi.FP8A_CENTER_K
    assert abi.prepare_workspace_bytes(big, cen) > abi.NOALLOC_SCRATCH_BYTES
    assert call(big, cen) == -5
    long_ctx = abi.make_shape(1, 32, 8, 32768, 128)                  # the 32k workload fits
    assert abi.prepare_workspace_bytes(long_ctx, cen) <= abi.NOALLOC_SCRATCH_BYTES
    assert abi.prepare_workspace_bytes(long_ctx, cen | abi.FP8A_TILE_SCALES) <= abi.NOALLOC_SCRATCH_BYTES
    assert call(abi.make_shape(1, 2, 1, 64, 96)) == -2
    assert call(abi.make_shape(1, 2, 1, 64, 64), flags=abi.FP8A_PREFIX_SCALES) == -4
    assert call(abi.make_shape(1, 2, 1, 64, 64), q=None) == -1
    assert call(abi.make_shape(1, 2, 1, 64, 64), flags=abi.FP8A_ROTATE_QK, signs=None) == -1
    assert f(None, 1, FAKE, FAKE, FAKE, 0, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, None) == -1


def test_noalloc_scratch_size_matches_the_header(abi):
    text = open(abi.HEADER).read()
    assert "#define FP8A_NOALLOC_SCRATCH_BYTES ((size_t)8 << 20)" in text
    assert abi.NOALLOC_SCRATCH_BYTES == 8 << 20


def test_fwd_rejects(abi):
    _no_gpu()
    ok = abi.make_shape(1, 2, 1, 64, 64)
    assert _fwd(abi, ok, bn=96) == -4
    assert _fwd(abi, ok, order=2) == -4
    assert _fwd(abi, ok, causal=3) == -4
    assert _fwd(abi, ok, scale=0.0) == -4
    assert _fwd(abi, ok, scale=float("nan")) == -4
    assert _fwd(abi, ok, S=0.0) == -4
    assert _fwd(abi, ok, S=500.0) == -4
    assert _fwd(abi, ok, S=100.0) == -3                                 # not a power of two nor 448
    assert _fwd(abi, ok, S=0.5) == -3
    assert _fwd(abi, ok, k_sink=-1) == -4
    assert _fwd(abi, ok, dtype=1) == -3                                 # bf16 operands go through prepare
    assert _fwd(abi, ok, dtype=4, desc=None) == -1                      # int8 Q/K codes need descales too
    assert _fwd(abi, ok, dtype=5) == -3
    assert _fwd(abi, ok, desc=None) == -1
    assert _fwd(abi, ok, out=None) == -1
    assert _fwd(abi, abi.make_shape(1, 2, 1, 64, 32)) == -2


def test_fwd_tile_scaled_rejects(abi):
    _no_gpu()
    ok = abi.make_shape(1, 2, 1, 64, 64)

    def call(shape=ok, desc=FAKE, out=FAKE, S=256.0, bn=128):
        return abi._lib.fp8_attn_fwd_tile_scaled(ctypes.byref(shape), FAKE, FAKE, FAKE, desc, desc, desc, 0.125, S,
                                                 1, bn, 1, out, None, None, None, None, 0, None)
    assert call(desc=None) == -1
    assert call(out=None) == -1
    assert call(S=100.0) == -3
    assert call(bn=32) == -4
    assert call(shape=abi.make_shape(1, 2, 1, 64, 32)) == -2


def test_head_error_rejects(abi):
    _no_gpu()
    ok = abi.make_shape(1, 2, 1, 64, 64)
    f = abi._lib.fp8_attn_head_error
    assert f(ctypes.byref(ok), FAKE, FAKE, 0, None, 63, FAKE, FAKE, 1 << 20, None) == -2   # nrows != N without rows
    assert f(ctypes.byref(ok), FAKE, FAKE, 1, None, 64, FAKE, FAKE, 1 << 20, None) == -3   # bf16 reference
    assert f(ctypes.byref(ok), None, FAKE, 0, None, 64, FAKE, FAKE, 1 << 20, None) == -1
    assert f(ctypes.byref(ok), FAKE, FAKE, 0, None, 64, FAKE, None, 0, None) == -5


def test_header_is_plain_c_and_links_from_c(tmp_path):
    """include/fp8_attn.h compiles as strict C99 and a C program links against
    the library and calls its host-side functions (no C++ or torch needed)."""
    import shutil
    import subprocess
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no C compiler")
    src = tmp_path / "caller.c"
    src.write_text(
        '#include <stdio.h>\n#include "fp8_attn.h"\n'
        "int main(void) {\n"
        "  fp8a_shape s = {1, 2, 1, 64, 64, {0, 0, 0}, {0, 0, 0}, {0, 0, 0}};\n"
        '  printf("%d %d\\n", fp8_attn_padded_seqlen(s.seqlen), (int)fp8_attn_prepare_workspace_bytes(&s, FP8A_ROTATE_QK) > 0);\n'
        "  return 0;\n}\n")
    exe = tmp_path / "caller"
    libdir = os.path.dirname(LIB)
    subprocess.run([gcc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", "-I", os.path.dirname(HEADER),
                    str(src), "-L", libdir, "-lfp8attn", "-Wl,-rpath," + libdir, "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split()
    assert out == ["128", "1"]


def _build_module():
    import importlib.util
    spec = importlib.util.spec_from_file_location(
        "_fp8attn_build_for_test", os.path.join(ROOT, "precision_attention_numerics_amd", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_library_built_from_these_sources(lib):
    """The in-tree library reports the hash of the sources it was compiled
    from; it must be the hash of the sources in this tree (a stale or foreign
    binary fails here)."""
    lib.fp8_attn_build_info.restype = ctypes.c_char_p
    info = lib.fp8_attn_build_info().decode()
    assert info == f"source_sha256={_build_module().source_hash()} arch=gfx950", info


def test_build_from_a_clean_checkout(tmp_path):
    """__graft_entry__.build() on the committed tree alone (git archive of
    HEAD: no built library, no working files) compiles the HIP library and the
    oracle, after which the package imports and the library reports the
    checkout's source hash."""
    import shutil
    import subprocess
    import sys
    if shutil.which("git") is None or not os.path.isdir(os.path.join(ROOT, ".git")):
        pytest.skip("needs the git repository")
    if shutil.which("/opt/rocm/bin/hipcc") is None and shutil.which("hipcc") is None:
        pytest.skip("needs hipcc")
    archive = subprocess.run(["git", "-C", ROOT, "archive", "HEAD"], check=True, capture_output=True).stdout
    subprocess.run(["tar", "-x", "-C", str(tmp_path)], input=archive, check=True)
    assert not os.path.exists(tmp_path / "precision_attention_numerics_amd" / "libfp8attn.so")
    code = ("import __graft_entry__ as g; g.build(); import precision_attention_numerics_amd as p, ctypes; "
            "p._abi._lib.fp8_attn_build_info.restype = ctypes.c_char_p; "
            "print('BUILD_INFO', p._abi._lib.fp8_attn_build_info().decode()); print('STATUS', p.strerror(0))")
    env = dict(os.environ, PYTHONDONTWRITEBYTECODE="1")
    res = subprocess.run([sys.executable, "-c", code], cwd=tmp_path, capture_output=True, text=True, timeout=900, env=env)
    assert res.returncode == 0, res.stderr[-3000:]
    lines = dict(l.split(" ", 1) for l in res.stdout.splitlines() if l.startswith(("BUILD_INFO", "STATUS")))
    assert lines["STATUS"] == "ok"
    import importlib.util
    spec = importlib.util.spec_from_file_location("_clean_build", tmp_path / "precision_attention_numerics_amd" / "build.py")
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    assert lines["BUILD_INFO"] == f"source_sha256={mod.source_hash()} arch=gfx950"
