"""One outer step on the GPU from a C program through the C ABI alone, with the
HIP runtime for device memory and no Python in the path (tests/c/gpu_step.c):
constant tensors against the exact Nesterov step, every used codebook entry of a
near-Gaussian tensor inside its bucket, and dlc_quantize_static equal to
dlc_quantize."""
import importlib.util
import os
import shutil
import subprocess

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "c", "gpu_step.c")
EXE = os.path.join(ROOT, "tests", "c", "gpu_step.bin")


def program():
    """The program __graft_entry__.build() compiled, or compiled here when missing
    or older than its source."""
    if os.path.exists(EXE) and os.path.getmtime(EXE) >= os.path.getmtime(SRC):
        return EXE
    if shutil.which("gcc") is None:
        pytest.skip("gcc is not installed and tests/c/gpu_step.bin was not built")
    spec = importlib.util.spec_from_file_location("dlc_build", os.path.join(ROOT, "diloco_outer_step_amd", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod.c_program(SRC, EXE)


def test_outer_step_from_c():
    exe = program()
    print(f"[c program] {exe}", flush=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    print(r.stdout, flush=True)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.startswith("ok "), r.stdout
