"""Build librmm.so (HIP, gfx950) in-tree.

Each ``csrc/*.hip`` translation unit is compiled separately with hipcc for
gfx950 and linked into ``input_adaptive_reduced_amd/librmm.so``.  Packed
fp32 vector instructions are disabled for every GPU compile.

``build(sanitize=True, out=...)`` makes a separate copy whose host code runs
under AddressSanitizer and UndefinedBehaviorSanitizer (GPU code unchanged),
for the host-side tests; it needs the clang sanitizer runtime loaded first.
"""
from __future__ import annotations

import concurrent.futures
import glob
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build", "librmm")
LIB_PATH = os.path.join(HERE, "librmm.so")
ARCH = "gfx950"

GPU_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
CXX_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-mcode-object-version=5", "-Wall", "-Wno-unused-result",
             "-I", INCLUDE, "-I", CSRC]
# host code only: each sanitizer flag right after -Xarch_host
HOST_SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer",
                 "-Xarch_host", "-g"]
HOST_SANITIZE_LINK = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", "-shared-libasan"]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 feature; that warning is expected
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{err}")
    return err


def build(verbose: bool = False, jobs: int = 4, sanitize: bool = False, out: str | None = None) -> str:
    """Compile every HIP source and link librmm.so; returns the library path.
    With ``sanitize`` the host code is instrumented and the library goes to
    ``out`` (required), objects to their own folder."""
    hipcc = _hipcc()
    if sanitize and not out:
        raise ValueError("a sanitized build needs its own output path")
    lib_path = out or LIB_PATH
    build_dir = BUILD_DIR + ("_sanitize" if sanitize else "")
    os.makedirs(build_dir, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    if not srcs:
        raise RuntimeError("no HIP sources found")
    objs = []
    extra = HOST_SANITIZE if sanitize else []

    def compile_one(src):
        obj = os.path.join(build_dir, os.path.basename(src) + ".o")
        cmd = [hipcc, "-c", src, "-o", obj] + CXX_FLAGS + GPU_FLAGS + extra
        warn = _run(cmd)
        if verbose and warn.strip():
            print(warn, file=sys.stderr)
        return obj

    with concurrent.futures.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(compile_one, srcs))
    tmp = lib_path + ".tmp%d" % os.getpid()
    _run([hipcc, "-shared", f"--offload-arch={ARCH}", "-mcode-object-version=5", "-o", tmp] + objs +
         (HOST_SANITIZE_LINK if sanitize else []))
    os.replace(tmp, lib_path)
    return lib_path


if __name__ == "__main__":
    print(build(verbose=True))
