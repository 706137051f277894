"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

libdlc_hostsan.so is libdlc.so with its host side (argument checks, fragment
plans, block partitions, ring plans, workspace layouts, launch orchestration)
instrumented; the device code is the same.  Two drivers exercise it on the CPU,
with no GPU and nothing launched:

  * the C99 program tests/c/abi_smoke.c (plans and workspace sizes of every
    call, the argument errors of every call that launches work), built and
    linked with the same sanitizers, leak detection on;
  * the host-only Python tests (exports, fragment plans against the oracle,
    argument errors, the binding's refusals) in a child process with the
    sanitizer runtime preloaded.

Any sanitizer report fails the run (recovery is off).
"""
import glob
import importlib.util
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "diloco_outer_step_amd")
LIB = os.path.join(PKG, "libdlc_hostsan.so")
CLANG = "/opt/rocm/llvm/bin/clang"


def hostsan_library():
    if not os.path.exists(LIB):
        spec = importlib.util.spec_from_file_location("dlc_build", os.path.join(PKG, "build.py"))
        mod = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(mod)
        mod.build(hostsan=True)
    return LIB


def asan_runtime():
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return found[-1] if found else None


pytestmark = pytest.mark.skipif(not os.path.exists(CLANG) or asan_runtime() is None,
                                reason="ROCm clang with the sanitizer runtimes is not installed")


def test_c_program_under_the_sanitizers(tmp_path):
    lib = hostsan_library()
    exe = tmp_path / "abi_smoke_san"
    cmd = [CLANG, "-std=c99", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "c", "abi_smoke.c"),
           "-L", PKG, f"-l:{os.path.basename(lib)}", f"-Wl,-rpath,{PKG}", "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:halt_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "Sanitizer" not in r.stderr and "runtime error" not in r.stderr, r.stderr
    assert "FAIL" not in r.stdout and r.stdout.count("ok") >= 40


def test_host_python_tests_under_the_sanitizers():
    lib = hostsan_library()
    env = dict(os.environ, LD_PRELOAD=asan_runtime(), DLC_LIBRARY=lib,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")
    cmd = [sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
           os.path.join(ROOT, "tests", "test_abi_host.py"), os.path.join(ROOT, "tests", "test_binding_checks.py"),
           "-k", "not without_its_library"]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=900, env=env, cwd=ROOT)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert "Sanitizer" not in r.stderr and "runtime error" not in r.stderr, r.stderr[-3000:]
    assert " passed" in r.stdout
