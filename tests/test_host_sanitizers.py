"""Host sanitizers on the C ABI layer (CPU only): api.hip's host code (argument validation, pyramid
geometry, workspace sizes and carving, launch set-up) is rebuilt with AddressSanitizer and
UndefinedBehaviorSanitizer, every flag behind -Xarch_host so only host code is instrumented (the
kernel objects are the regular build's).  The host-side ABI tests then run against that library in
a child process that preloads the toolchain's ASan runtime; any report fails the child.

No kernel runs: the ABI tests call only size queries and argument checks that return before
anything is enqueued.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

import pytest

from hierarchical_top_selection_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HOST_SANITIZE = ["-O1", "-fno-omit-frame-pointer"] + [
    x for f in ("-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=undefined")
    for x in ("-Xarch_host", f)]


def rocm_dir() -> str:
    return os.path.dirname(os.path.dirname(os.path.realpath(B._hipcc())))


def asan_runtime() -> str | None:
    """The toolchain's shared ASan runtime (it carries the UBSan handlers too)."""
    for pattern in ("llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so",
                    "llvm/lib/clang/*/lib/x86_64-unknown-linux-gnu/libclang_rt.asan.so"):
        found = sorted(glob.glob(os.path.join(rocm_dir(), pattern)))
        if found:
            return found[-1]
    return None


def build_host_sanitized(out_dir: str) -> str:
    hipcc = B._hipcc()
    os.makedirs(B.BUILD_DIR, exist_ok=True)
    objs = []
    for name in sorted(os.listdir(B.CSRC)):
        if not name.endswith(".hip") or name == "api.hip":
            continue
        src = os.path.join(B.CSRC, name)
        obj = os.path.join(B.BUILD_DIR, name + ".o")
        fresh = os.path.exists(obj) and os.path.getmtime(obj) >= max(
            os.path.getmtime(p) for p in glob.glob(os.path.join(B.CSRC, "*")))
        objs.append(obj if fresh else B._compile(src, hipcc, False))
    api_obj = os.path.join(out_dir, "api_hostsan.o")
    flags = [f for f in B.FLAGS if f != "-O3"]
    res = subprocess.run([hipcc, *flags, *HOST_SANITIZE, "-c", os.path.join(B.CSRC, "api.hip"), "-o", api_obj],
                         capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-3000:]
    lib = os.path.join(out_dir, "libpisa.so")
    rocm_lib = os.path.join(rocm_dir(), "lib")
    res = subprocess.run([os.path.join(rocm_dir(), "llvm", "bin", "clang++"), "-shared", "-shared-libasan",
                          "-fsanitize=address,undefined", api_obj, *objs, f"-L{rocm_lib}", "-lamdhip64",
                          f"-Wl,-rpath,{rocm_lib}", "-o", lib], capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-3000:]
    return lib


def test_abi_host_code_is_clean_under_asan_and_ubsan(tmp_path):
    runtime = asan_runtime()
    if runtime is None:
        pytest.skip("the toolchain has no shared ASan runtime")
    lib = build_host_sanitized(str(tmp_path))
    code = ("import sys; sys.path[:0] = [%r, %r]\n"
            "from hierarchical_top_selection_amd import binding\n"
            "binding.LIB_PATH = %r; binding._lib = None\n"
            "import pytest\n"
            "sys.exit(pytest.main(['-q', '-m', 'not gpu', '-p', 'no:cacheprovider', %r]))\n"
            % (ROOT, os.path.join(ROOT, "tests"), lib, os.path.join(ROOT, "tests", "test_abi.py")))
    env = dict(os.environ, LD_PRELOAD=runtime, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([sys.executable, "-c", code], env=env, cwd=ROOT, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert " passed" in out, out[-2000:]
