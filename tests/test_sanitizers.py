"""The oracle's C code and the library's host-side entry points under
AddressSanitizer + UndefinedBehaviorSanitizer (CPU only).

Both are rebuilt with the sanitizers (oracle/build.py --sanitize;
precision_attention_numerics_amd/build.py --sanitize, which instruments the
host pass of abi.hip only) and the CPU tests that exercise them run in a
child process with the clang sanitizer runtime preloaded and FP8A_ORACLE_LIB /
FP8A_LIB pointing at the sanitized builds.  Any sanitizer report aborts the
child.  A planted out-of-bounds read, built with the same flags, shows the
set-up catches errors at all."""
import importlib.util
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
TESTS = ["test_abi_cpu.py", "test_oracle_codec.py", "test_oracle_emulator.py", "test_oracle_exp.py",
         "test_oracle_exp_table.py", "test_oracle_fwht.py", "test_oracle_ideal.py", "test_oracle_int8.py",
         "test_oracle_pcast.py", "test_oracle_rowhash.py", "test_oracle_tilescale.py"]
REPORTS = ("ERROR: AddressSanitizer", "runtime error:", "ERROR: LeakSanitizer")


def _module(name, path):
    spec = importlib.util.spec_from_file_location(name, path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


@pytest.fixture(scope="module")
def san():
    ob = _module("_oracle_build", os.path.join(ROOT, "oracle", "build.py"))
    lb = _module("_lib_build", os.path.join(ROOT, "precision_attention_numerics_amd", "build.py"))
    olib = ob.build(sanitize=True)
    llib = lb.build_sanitized()
    env = dict(os.environ, LD_PRELOAD=lb.san_runtime(), FP8A_ORACLE_LIB=olib, FP8A_LIB=llib,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    return ob, lb, env


def test_planted_overflow_is_reported(san, tmp_path):
    ob, lb, env = san
    src = tmp_path / "oob.c"
    src.write_text("#include <stdlib.h>\nint main(int c, char** v) { int* a = malloc(4 * sizeof(int));\n"
                   "  int r = a[c + 3]; free(a); return r; }\n")
    exe = tmp_path / "oob"
    subprocess.run([ob.SAN_CC, "-O0", *[f for f in ob.SAN_FLAGS if f != "-shared-libasan"], "-shared-libasan",
                    "-o", str(exe), str(src)], check=True)
    res = subprocess.run([str(exe)], env=env, capture_output=True, text=True, timeout=60)
    assert res.returncode != 0 and "heap-buffer-overflow" in res.stderr


@pytest.mark.timeout(900)
def test_cpu_suite_under_sanitizers(san):
    ob, lb, env = san
    cmd = [sys.executable, "-m", "pytest", "-q", "-x", "-m", "not gpu", "-p", "no:cacheprovider",
           "--deselect", "tests/test_abi_cpu.py::test_build_from_a_clean_checkout"]
    cmd += [os.path.join("tests", t) for t in TESTS]
    res = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=840)
    out = res.stdout + res.stderr
    print(out[-1500:])
    assert not any(r in out for r in REPORTS), "sanitizer report"
    assert res.returncode == 0, out[-3000:]
    # the child really ran on the sanitized builds
    probe = subprocess.run([sys.executable, "-c",
                            "import oracle, precision_attention_numerics_amd; oracle._load(); "
                            "m = open('/proc/self/maps').read(); "
                            "print('liboracle_san.so' in m, 'libfp8attn_san.so' in m)"],
                           cwd=ROOT, env=env, capture_output=True, text=True, timeout=120)
    assert probe.stdout.split() == ["True", "True"], probe.stdout + probe.stderr
