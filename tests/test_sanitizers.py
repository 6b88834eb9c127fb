"""Host code under sanitizers (CPU only, no GPU work).

* The C oracle with AddressSanitizer + UndefinedBehaviorSanitizer, and with
  ThreadSanitizer (its product splits rows over POSIX threads), driven by
  tests/sanitize_oracle.c.
* librmm's host code (argument checks, plans, workspace sizing of every entry
  point) built with AddressSanitizer + UndefinedBehaviorSanitizer on the host
  side only, driven by tests/sanitize_host.cpp, which makes only calls that
  return before any GPU work.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests")
OUT = os.path.join(ROOT, "_build", "sanitize")
CLANG = "/opt/rocm/llvm/bin/clang"
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=0",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
           "TSAN_OPTIONS": "halt_on_error=1"}


def run(cmd, env=None, timeout=300):
    e = dict(os.environ)
    e.update(SAN_ENV)
    if env:
        e.update(env)
    return subprocess.run(cmd, capture_output=True, text=True, env=e, timeout=timeout)


def build_oracle_driver(kind):
    if shutil.which("gcc") is None:
        pytest.skip("gcc is not installed")
    os.makedirs(OUT, exist_ok=True)
    exe = os.path.join(OUT, f"oracle_{kind}")
    san = ["-fsanitize=address,undefined"] if kind == "asan" else ["-fsanitize=thread"]
    cmd = ["gcc", "-std=c11", "-D_GNU_SOURCE", "-O1", "-g", "-fno-omit-frame-pointer", "-ffp-contract=off",
           "-fno-sanitize-recover=all", *san, os.path.join(HERE, "sanitize_oracle.c"),
           os.path.join(ROOT, "oracle", "rmm_oracle.c"), "-o", exe, "-lm", "-pthread"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return exe


@pytest.mark.parametrize("kind", ["asan", "tsan"])
def test_oracle_under_sanitizers(kind):
    exe = build_oracle_driver(kind)
    r = run([exe])
    if kind == "tsan" and "unexpected memory mapping" in r.stderr:
        pytest.skip("ThreadSanitizer cannot map its shadow memory in this environment")
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout + r.stderr


def test_library_host_code_under_sanitizers():
    if not os.path.exists(CLANG):
        pytest.skip("the ROCm clang is not installed")
    from input_adaptive_reduced_amd.build import build
    os.makedirs(OUT, exist_ok=True)
    lib = build(jobs=6, sanitize=True, out=os.path.join(OUT, "librmm.so"))
    rt = subprocess.run([CLANG, "--print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True,
                        text=True).stdout.strip()
    assert os.path.exists(rt), rt
    exe = os.path.join(OUT, "abi_host")
    cmd = [CLANG + "++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-shared-libasan", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
           "-I", "/opt/rocm/include", os.path.join(HERE, "sanitize_host.cpp"), lib, "-o", exe,
           f"-Wl,-rpath,{OUT}", f"-Wl,-rpath,{os.path.dirname(rt)}"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = run([exe])
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout + r.stderr
