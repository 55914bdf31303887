"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

``api.cpp`` (descriptor and argument validation, workspace planning, the
timer, the static-scratch bookkeeping) is rebuilt with both sanitizers on the
host side only and linked with the device objects of the normal build
(``_build/``, written by ``build()``); a child process then runs the ABI tests
against that library (``SIKV_LIBRARY``), with the sanitizer runtime preloaded,
so any invalid memory access or undefined behaviour on those paths aborts it.
No GPU is used: every call there fails a host check before a launch.  The
no-mutable-globals check is left out of that run (the sanitizer adds writable
globals of its own).
"""

import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BUILD = os.path.join(ROOT, "_build")
DEVICE_OBJS = ["encode.o", "score.o", "attn.o", "dense.o", "util.o"]


def _hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    return None


def _asan_runtime():
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return found[-1] if found else None


def test_abi_checks_under_host_sanitizers(tmp_path):
    hipcc, rt = _hipcc(), _asan_runtime()
    objs = [os.path.join(BUILD, o) for o in DEVICE_OBJS]
    if hipcc is None or rt is None:
        pytest.skip("hipcc or the sanitizer runtime is not installed")
    if not all(os.path.exists(o) for o in objs):
        pytest.skip("no device objects in _build/ (run build() first)")
    obj = str(tmp_path / "api_san.o")
    lib = str(tmp_path / "libsikv_san.so")
    compile_cmd = [
        hipcc, "-x", "hip", "-O1", "-g", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
        "-mcode-object-version=5", "-ffp-contract=off",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", os.path.join(ROOT, "include"),
        "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
        "-Xarch_host", "-fno-sanitize-recover=undefined",
        "-Xarch_host", "-fno-omit-frame-pointer",
        "-c", os.path.join(ROOT, "bit_self_indexed_amd", "csrc", "api.cpp"), "-o", obj]
    r = subprocess.run(compile_cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-3000:]
    link_cmd = [hipcc, "-shared", "-fPIC", "--offload-arch=gfx950", obj, *objs, "-o", lib]
    r = subprocess.run(link_cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ)
    env["SIKV_LIBRARY"] = lib
    # the runtime must come first among preloaded libraries; any others stay
    env["LD_PRELOAD"] = rt + (":" + env["LD_PRELOAD"] if env.get("LD_PRELOAD") else "")
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    run = subprocess.run(
        [sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi.py"), "-q",
         "-m", "not gpu", "-p", "no:cacheprovider", "-k", "not mutable_globals"],
        capture_output=True, text=True, timeout=900, cwd=ROOT, env=env)
    tail = (run.stdout + run.stderr)[-4000:]
    assert run.returncode == 0, tail
    assert " passed" in run.stdout and "failed" not in run.stdout, tail
