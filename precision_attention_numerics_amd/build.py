"""Builds the HIP library libfp8attn.so for gfx950 (in-tree, next to this file).

Each source is compiled to an object in parallel, then the objects are linked.
This module is importable without the package (it imports nothing from it), so
a fresh checkout can build before the library exists.
"""
import concurrent.futures
import hashlib
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
SOURCES = ["abi.hip", "prepare.hip", "attn_fwd.hip", "attn_fwd32.hip", "head_error.hip"]
LIB = os.path.join(HERE, "libfp8attn.so")
OBJDIR = os.path.join(ROOT, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

COMPILE_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # every binary32 operation on the P path is an explicit single operation
    "-ffp-contract=off",
    # no packed FP32 VALU instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]
# a symbol left undefined (e.g. a kernel launch stub the host pass did not
# emit) fails the build instead of the first load
LINK_FLAGS = ["--offload-arch=gfx950", "-shared", "-fPIC", "-Wl,--no-undefined"]
# Host-side AddressSanitizer + UndefinedBehaviorSanitizer build of the entry
# points (argument validation, workspace layout, launch set-up): abi.hip is
# recompiled with the sanitizers on its host pass only (device code is never
# instrumented) and linked with the other objects into SAN_LIB, which needs
# the clang sanitizer runtime preloaded (SAN_RUNTIME).
SAN_LIB = os.path.join(HERE, "libfp8attn_san.so")
SAN_HOST_FLAGS = []
for _f in ("-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"):
    SAN_HOST_FLAGS += ["-Xarch_host", _f]
SAN_LINK_FLAGS = ["-shared-libasan", "-fsanitize=address,undefined"]


def san_runtime() -> str:
    """The clang AddressSanitizer runtime the sanitized builds link against."""
    import glob
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not found:
        raise FileNotFoundError("libclang_rt.asan-x86_64.so not found under /opt/rocm/llvm")
    return found[-1]


def source_files() -> list[str]:
    """Every file the library is built from (sources, headers, this script)."""
    files = [os.path.join(CSRC, f) for f in sorted(os.listdir(CSRC)) if f.endswith((".hip", ".hpp"))]
    files.append(os.path.join(ROOT, "include", "fp8_attn.h"))
    files.append(os.path.abspath(__file__))
    return files


def source_hash() -> str:
    h = hashlib.sha256()
    for f in source_files():
        h.update(os.path.basename(f).encode())
        h.update(open(f, "rb").read())
    return h.hexdigest()


def _filter(stderr: str) -> str:
    return "\n".join(l for l in stderr.splitlines()
                     if "packed-fp32-ops" not in l and "unknown target feature" not in l)


def _compile(src: str, obj: str, extra: list[str]) -> tuple[str, int, str]:
    cmd = [HIPCC] + COMPILE_FLAGS + extra + ["-c", "-o", obj, src]
    res = subprocess.run(cmd, capture_output=True, text=True)
    return " ".join(cmd), res.returncode, _filter(res.stderr)


def build_sanitized(verbose: bool = False) -> str:
    """SAN_LIB: abi.hip with host sanitizers, the kernels as in the normal build."""
    digest = source_hash()
    objs = [os.path.join(OBJDIR, s.replace(".hip", ".o")) for s in SOURCES if s != "abi.hip"]
    if not all(os.path.exists(o) for o in objs):
        build(verbose)
    extra = [f"-DFP8A_SOURCE_SHA256=\"{digest}\""] + SAN_HOST_FLAGS
    san_obj = os.path.join(OBJDIR, "abi_san.o")
    cmd, rc, err = _compile(os.path.join(CSRC, "abi.hip"), san_obj, extra)
    if verbose:
        print(cmd, flush=True)
    if rc != 0:
        raise RuntimeError(f"hipcc failed ({rc}):\n{cmd}\n{err}")
    cmd = [HIPCC] + LINK_FLAGS + SAN_LINK_FLAGS + ["-o", SAN_LIB + ".tmp", san_obj] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc link failed ({res.returncode}):\n{_filter(res.stderr)}")
    os.replace(SAN_LIB + ".tmp", SAN_LIB)
    return SAN_LIB


def build(verbose: bool = False) -> str:
    os.makedirs(OBJDIR, exist_ok=True)
    digest = source_hash()
    # the library reports the hash of the sources it was built from
    extra = [f"-DFP8A_SOURCE_SHA256=\"{digest}\""]
    jobs = []
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1)) as ex:
        for s in SOURCES:
            obj = os.path.join(OBJDIR, s.replace(".hip", ".o"))
            jobs.append(ex.submit(_compile, os.path.join(CSRC, s), obj, extra))
        for j in jobs:
            cmd, rc, err = j.result()
            if verbose:
                print(cmd, flush=True)
            if rc != 0:
                raise RuntimeError(f"hipcc failed ({rc}):\n{cmd}\n{err}")
            if verbose and err.strip():
                print(err)
    objs = [os.path.join(OBJDIR, s.replace(".hip", ".o")) for s in SOURCES]
    cmd = [HIPCC] + LINK_FLAGS + ["-o", LIB + ".tmp"] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc link failed ({res.returncode}):\n{_filter(res.stderr)}")
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    if "--sanitize" in sys.argv:
        build_sanitized(verbose="-v" in sys.argv)
    else:
        build(verbose="-v" in sys.argv)
