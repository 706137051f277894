"""Build the gfx950 shared library libdlc.so in-tree with hipcc.

    python diloco_outer_step_amd/build.py          # libdlc.so
    python diloco_outer_step_amd/build.py hostsan  # also libdlc_hostsan.so

(run as a script: importing the package needs the library that this script compiles)

Each source compiles to an object under _build/ (the two in parallel), then the
objects link into the library.  libdlc_hostsan.so is the same library with its
host code (argument checks, fragment plans, block partitions, workspace layouts,
launch orchestration) built with AddressSanitizer and UndefinedBehaviorSanitizer;
the device code is not instrumented.  The CPU tests drive it from a C program
linked with the same sanitizers.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJ = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libdlc.so")
LIB_HOSTSAN = os.path.join(PKG, "libdlc_hostsan.so")
SOURCES = ["dlc_api.hip", "dlc_kernels.hip"]
ARCH = "gfx950"

FLAGS = [
    "-O3", "-std=c++17", "-fPIC",
    f"--offload-arch={ARCH}",
    # no fused multiply-add unless written explicitly: results must match the IEEE
    # definition of every step bit for bit
    "-ffp-contract=off",
    # keep packed-fp32 instructions out of generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
]
# Host-side sanitizers only: each flag applies to the host compilation.
HOSTSAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer", "-g"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    return "hipcc"


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)


def _compile(src: str, obj: str, extra, verbose: bool) -> str:
    _run([hipcc(), *FLAGS, *extra, f"-I{INCLUDE}", f"-I{CSRC}", "-c", os.path.join(CSRC, src), "-o", obj], verbose)
    return obj


def _link(objs, out: str, verbose: bool, sanitize: bool = False) -> str:
    tmp = out + ".tmp"
    if sanitize:
        # objects already carry their device code: the host linker, with the
        # sanitizer runtimes, links them against the HIP runtime
        rocm = os.path.dirname(os.path.dirname(os.path.realpath(hipcc())))
        cmd = [os.path.join(rocm, "llvm", "bin", "clang++"), "-shared", "-fsanitize=address,undefined", *objs,
               f"-L{rocm}/lib", "-lamdhip64", f"-Wl,-rpath,{rocm}/lib"]
    else:
        cmd = [hipcc(), "-shared", f"--offload-arch={ARCH}", *objs]
    _run([*cmd, "-o", tmp], verbose)
    os.replace(tmp, out)
    return out


def c_program(src: str, out: str, verbose: bool = False) -> str:
    """Compile a C99 program that calls the C ABI and the HIP runtime (gcc, linked
    against libdlc.so and libamdhip64 with run paths to both)."""
    rocm = os.path.dirname(os.path.dirname(os.path.realpath(hipcc())))
    _run(["gcc", "-std=c99", "-O2", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__", f"-I{rocm}/include",
          f"-I{INCLUDE}", src, f"-L{PKG}", "-l:libdlc.so", f"-L{rocm}/lib", "-lamdhip64", "-lm",
          f"-Wl,-rpath,{PKG}", f"-Wl,-rpath,{rocm}/lib", "-o", out + ".tmp"], verbose)
    os.replace(out + ".tmp", out)
    return out


def build(verbose: bool = False, hostsan: bool = True) -> str:
    """Compile every HIP source and link libdlc.so (always recompiles); with
    hostsan, also the host-sanitized libdlc_hostsan.so."""
    os.makedirs(OBJ, exist_ok=True)
    jobs = [(s, os.path.join(OBJ, s.replace(".hip", ".o")), []) for s in SOURCES]
    if hostsan:
        jobs.append(("dlc_api.hip", os.path.join(OBJ, "dlc_api_hostsan.o"), HOSTSAN))
    with ThreadPoolExecutor(len(jobs)) as ex:
        objs = list(ex.map(lambda j: _compile(*j, verbose), jobs))
    _link(objs[:2], LIB, verbose)
    if hostsan:
        _link([objs[2], objs[1]], LIB_HOSTSAN, verbose, sanitize=True)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, hostsan="hostsan" in sys.argv))
