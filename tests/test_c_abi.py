"""The C ABI from plain C: include/dlc.h compiles as C99 with gcc, a C program
links against libdlc.so and runs the host-only calls and argument checks (no
GPU needed)."""
import os
import shutil
import subprocess

import pytest

import diloco_outer_step_amd as dlc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc is not installed")
def test_c_program_uses_the_abi(tmp_path):
    exe = tmp_path / "abi_smoke"
    libdir = os.path.dirname(dlc.LIB_PATH)
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "c", "abi_smoke.c"), "-L", libdir, "-ldlc", f"-Wl,-rpath,{libdir}",
           "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "FAIL" not in r.stdout and r.stdout.count("ok") >= 12


def test_last_error_is_per_thread():
    import threading
    results = {}

    def fail_here():
        with pytest.raises(dlc.DlcError):
            dlc.dlc_workspace_bytes(0, [(0, 0, 64)])
        results["other"] = dlc.dlc_last_error()

    with pytest.raises(dlc.DlcError):
        dlc.dlc_workspace_bytes(65, [(0, 0, 64)])
    mine = dlc.dlc_last_error()
    th = threading.Thread(target=fail_here)
    th.start()
    th.join()
    # the other thread's failure did not overwrite this thread's message, and a
    # successful call clears only its own thread's message
    assert dlc.dlc_last_error() == mine and results["other"] != ""
    dlc.dlc_workspace_bytes(1, [(0, 0, 64)])
    assert dlc.dlc_last_error() == ""
