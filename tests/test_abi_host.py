"""Host-side checks of the C ABI (no GPU needed, nothing is launched).

* libdlc.so loads and exports every function include/dlc.h declares;
* dlc_fragment_plan (C++) equals the oracle's greedy bin-packing on every
  parameter set, tensor for tensor;
* every argument error is reported with its status code before any launch.
"""
import ctypes
import os
import re

import numpy as np
import pytest

import diloco_outer_step_amd as dlc
import oracle
import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dlc.h")

FAKE = 1 << 20  # a 256-byte aligned address that is never dereferenced (calls fail first)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dlc_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    names = declared_functions()
    assert len(names) >= 8
    lib = ctypes.CDLL(dlc.LIB_PATH)
    for name in names:
        assert hasattr(lib, name), f"{name} declared in dlc.h but not exported"
    assert set(names) == set(dlc.EXPORTED)
    assert "gfx950" in dlc.dlc_version()


def test_header_constants_match_binding():
    text = open(HEADER).read()
    for name in ("DLC_OK", "DLC_ERR_INVALID_ARGUMENT", "DLC_ERR_ALIGNMENT", "DLC_ERR_NO_QUORUM",
                 "DLC_ERR_WORKSPACE", "DLC_ERR_HIP", "DLC_MAX_LEARNERS", "DLC_N_BUCKETS",
                 "DLC_ALIGN_ELEMS", "DLC_RANGE_FIELDS", "DLC_RANGE_GIVEN", "DLC_BROADCAST", "DLC_TWO_LANES",
                 "DLC_MAX_LANES", "DLC_ERR_NON_FINITE", "DLC_DEBUG_CHECKS", "DLC_STATIC_SCRATCH_BYTES"):
        m = re.search(rf"#define {name} \(?(-?\d+)u?\)?", text)
        assert m and int(m.group(1)) == getattr(dlc, name), name


@pytest.mark.parametrize("key", ["c2", "c3", "c4", "c5k1"])
@pytest.mark.parametrize("p", [1, 7, 24])
def test_fragment_plan_matches_oracle(key, p):
    numel = [s.numel for s in workloads.config(key).tensors]
    got = dlc.dlc_fragment_plan(numel, p)
    want = oracle.fragment_plan(numel, p)
    assert got[0] == list(want[0])
    assert got[1] == list(want[1])


def test_fragment_plan_random_with_ties():
    # sizes drawn from few values, so equal sizes and equal loads are common and the
    # tie rules (equal sizes in index order, equal loads to the lowest fragment) decide
    rng = np.random.default_rng(5)
    for case in range(300):
        n = int(rng.integers(1, 60))
        pool = rng.integers(1, 5000, int(rng.integers(1, 6)))
        numel = [int(x) for x in rng.choice(pool, n)]
        p = int(rng.integers(1, 30))
        assert dlc.dlc_fragment_plan(numel, p) == oracle.fragment_plan(numel, p), (case, numel, p)


def test_fragment_plan_small_cases():
    assert dlc.dlc_fragment_plan([7, 5, 4, 3, 3, 2], 2) == ([0, 1, 1, 0, 1, 0], [12, 12])
    assert dlc.dlc_fragment_plan([5, 1], 4) == ([0, 1], [5, 1, 0, 0])
    with pytest.raises(dlc.DlcError):
        dlc.dlc_fragment_plan([3, 0], 2)
    with pytest.raises(dlc.DlcError):
        dlc.dlc_fragment_plan([3], 0)


def test_workspace_bytes_grows_with_learners():
    t = [(0, 0, 1 << 22), (1 << 22, 1 << 22, 4096)]
    a = dlc.dlc_workspace_bytes(1, t)
    b = dlc.dlc_workspace_bytes(16, t)
    assert 0 < a < b and a % 256 == 0 and b % 256 == 0
    with pytest.raises(dlc.DlcError):
        dlc.dlc_workspace_bytes(0, t)


# --- argument errors: every call returns its status before touching the GPU ----------

L = dlc._lib


def tens(spec):
    arr = (dlc._Tensor * max(1, len(spec)))()
    for i, (o, lo, n) in enumerate(spec):
        arr[i].offset, arr[i].loffset, arr[i].numel = o, lo, n
    return arr, len(spec)


def quantize(k=2, spec=((0, 0, 4096),), stride=4096, theta=FAKE, present=None, ws_bytes=1 << 30,
             ws=FAKE, codes=FAKE, flags=0):
    arr, n = tens(spec)
    pres = None
    if present is not None:
        buf = (ctypes.c_uint8 * k)(*present)
        pres = ctypes.cast(buf, ctypes.c_void_p)
    return L.dlc_quantize(theta, FAKE, stride, k, pres, arr, n, codes, FAKE, FAKE, flags, ws, ws_bytes, None)


def quantize_static(k=2, spec=((0, 0, 4096),), stride=4096, present=None, flags=0):
    """dlc_quantize_static with fake pointers: only calls whose arguments or scratch
    size are refused before the device is touched belong here."""
    arr, n = tens(spec)
    pres = None
    if present is not None:
        buf = (ctypes.c_uint8 * k)(*present)
        pres = ctypes.cast(buf, ctypes.c_void_p)
    return L.dlc_quantize_static(FAKE, FAKE, stride, k, pres, arr, n, FAKE, FAKE, FAKE, flags, None)


# a call whose workspace exceeds the static scratch: one tensor of 2^27 elements
# (8192 encode blocks of 4 tiles) with 16 learners needs 256 MiB of histograms
BIG_STATIC = dict(k=16, spec=((0, 0, 1 << 27),), stride=1 << 27)


def quantize_bases(bases=(FAKE, FAKE), present=None, ws_bytes=16):
    """ws_bytes=16 is too small, so a call that passes every other check stops at
    the workspace check instead of launching."""
    L = dlc._lib
    arr, n = dlc._tensors(((0, 0, 4096),))
    ptrs = None if bases is None else ctypes.cast((ctypes.c_void_p * 2)(*bases), ctypes.c_void_p)
    pres = None if present is None else ctypes.cast((ctypes.c_uint8 * 2)(*present), ctypes.c_void_p)
    return L.dlc_quantize_bases(ptrs, FAKE, 4096, 2, pres, arr, n, FAKE, FAKE, FAKE, FAKE, ws_bytes, None)


def broadcast(k=2, spec=((0, 0, 4096),), stride=4096, theta=FAKE):
    L = dlc._lib
    arr, n = dlc._tensors(spec)
    return L.dlc_broadcast(theta, FAKE, stride, k, None, arr, n, None)


def cycle_ws(k=2, spec=((0, 0, 4096), (4096, 4096, 64)), first=(0, 1, 2)):
    L = dlc._lib
    arr, _ = dlc._tensors(spec)
    fb = (ctypes.c_int32 * len(first))(*first)
    out = ctypes.c_size_t(0)
    return L.dlc_cycle_workspace_bytes(k, arr, ctypes.cast(fb, ctypes.c_void_p), len(first) - 1, ctypes.byref(out))


def cycle(k=2, spec=((0, 0, 4096), (4096, 4096, 64)), first=(0, 1, 2), stride=8192,
          weights=((1.0, 1.0), (1.0, 1.0)), flags=0, ws_bytes=1 << 30, codes=FAKE):
    L = dlc._lib
    arr, _ = dlc._tensors(spec)
    fb = (ctypes.c_int32 * len(first))(*first)
    w = (ctypes.c_double * (len(weights) * k))(*[x for row in weights for x in row])
    return L.dlc_outer_cycle(FAKE, FAKE, FAKE, stride, k, ctypes.cast(w, ctypes.c_void_p), arr,
                             ctypes.cast(fb, ctypes.c_void_p), len(first) - 1, codes, FAKE, FAKE, 0.7, 0.9, flags,
                             FAKE, ws_bytes, None, None)


def cycle_lanes(n_lanes=3, streams=True, flags=0, ws_bytes=1 << 30, weights=((1.0, 1.0), (1.0, 1.0))):
    L = dlc._lib
    k, spec, first = 2, ((0, 0, 4096), (4096, 4096, 64)), (0, 1, 2)
    arr, _ = dlc._tensors(spec)
    fb = (ctypes.c_int32 * len(first))(*first)
    w = (ctypes.c_double * (len(weights) * k))(*[x for row in weights for x in row])
    ss = (ctypes.c_void_p * 9)()  # null streams: the calls below fail before anything is enqueued
    return L.dlc_outer_cycle_lanes(FAKE, FAKE, FAKE, 8192, k, ctypes.cast(w, ctypes.c_void_p), arr,
                                   ctypes.cast(fb, ctypes.c_void_p), len(first) - 1, FAKE, FAKE, FAKE, 0.7, 0.9,
                                   flags, FAKE, ws_bytes, ctypes.cast(ss, ctypes.c_void_p) if streams else None,
                                   n_lanes)


def lanes_ws_short():
    """Workspace for two lanes handed to a call with three."""
    arr, _ = dlc._tensors(((0, 0, 4096), (4096, 4096, 64)))
    need = dlc.dlc_cycle_workspace_bytes(2, ((0, 0, 4096), (4096, 4096, 64)), (0, 1, 2))
    return cycle_lanes(n_lanes=3, ws_bytes=2 * need)


def merge(k=2, spec=((0, 0, 4096),), stride=4096, weights=(1.0, 1.0), lr=0.7, beta=0.9, flags=0, theta=FAKE):
    arr, n = tens(spec)
    w = (ctypes.c_double * k)(*weights)
    return L.dlc_merge_outer_step(theta, FAKE, FAKE, stride, k, FAKE, ctypes.cast(w, ctypes.c_void_p), arr, n,
                                  lr, beta, flags, None)


def ring(k=2, spec=((0, 0, 4096),), stride=4096, lr=0.7, ws_bytes=16, accum=FAKE):
    """ws_bytes=16 stops a call that passes every other check at the workspace check."""
    arr, n = tens(spec)
    return L.dlc_ring_outer_step(FAKE, FAKE, FAKE, stride, k, arr, n, lr, 0.9, accum, FAKE, FAKE, FAKE, FAKE,
                                 ws_bytes, None)


def rda(k=2, spec=((0, 0, 4096),), stride=4096, weights=(1.0, 1.0), norms=FAKE, ws_bytes=16, theta=FAKE):
    arr, n = tens(spec)
    w = (ctypes.c_double * k)(*weights)
    return L.dlc_rda_outer_step(theta, FAKE, FAKE, None, stride, k, arr, n, ctypes.cast(w, ctypes.c_void_p), 0.7,
                                0.9, FAKE, FAKE, FAKE, norms, FAKE, ws_bytes, None)


@pytest.mark.parametrize("call,code", [
    (lambda: ring(k=0), dlc.DLC_ERR_INVALID_ARGUMENT),
    (lambda: ring(accum=None), dlc.DLC_ERR_INVALID_ARGUMENT),
    (lambda: ring(accum=FAKE + 4), dlc.DLC_ERR_ALIGNMENT),
    (lambda: ring(lr=float("nan")), dlc.DLC_ERR_INVALID_ARGUMENT),
    (lambda: ring(stride=100), dlc.DLC_ERR_ALIGNMENT),
    (lambda: ring(), dlc.DLC_ERR_WORKSPACE),
    (lambda: rda(weights=(0.0, 0.0)), dlc.DLC_ERR_NO_QUORUM),
    (lambda: rda(weights=(1.0, -1.0)), dlc.DLC_ERR_INVALID_ARGUMENT),
    (lambda: rda(norms=None), dlc.DLC_ERR_INVALID_ARGUMENT),
    (lambda: rda(norms=FAKE + 8), dlc.DLC_ERR_ALIGNMENT),
    (lambda: rda(theta=FAKE + 4), dlc.DLC_ERR_ALIGNMENT),
    (lambda: rda(spec=((0, 0, 0),)), dlc.DLC_ERR_INVALID_ARGUMENT),
    (lambda: rda(k=65, weights=(1.0,) * 65), dlc.DLC_ERR_INVALID_ARGUMENT),
    (lambda: rda(), dlc.DLC_ERR_WORKSPACE),
])
def test_ring_and_rda_argument_errors(call, code):
    assert call() == code
    assert dlc.dlc_last_error() != ""


@pytest.mark.parametrize("call", [
    lambda: quantize(spec=()),
    lambda: merge(spec=()),
    lambda: ring(spec=()),
    lambda: rda(spec=()),
    lambda: broadcast(spec=()),
])
def test_a_call_without_tensors_is_an_argument_error(call):
    assert call() == dlc.DLC_ERR_INVALID_ARGUMENT
    assert "n_tensors" in dlc.dlc_last_error()


def test_rda_and_ring_workspace_sizes():
    t = [(0, 0, 1 << 22), (1 << 22, 1 << 22, 4096)]
    q = dlc.dlc_workspace_bytes(4, t)
    r = dlc.dlc_rda_workspace_bytes(4, t)
    assert r > q and r % 256 == 0
    assert dlc.dlc_ring_workspace_bytes(4, t) > 0
    with pytest.raises(dlc.DlcError):
        dlc.dlc_rda_workspace_bytes(0, t)


@pytest.mark.parametrize("call,code", [
    (lambda: quantize(k=0), dlc.DLC_ERR_INVALID_ARGUMENT),
    (lambda: quantize(k=65), dlc.DLC_ERR_INVALID_ARGUMENT),
    (lambda: quantize(theta=None), dlc.DLC_ERR_INVALID_ARGUMENT),
    (lambda: quantize(theta=FAKE + 4), dlc.DLC_ERR_ALIGNMENT),
    (lambda: quantize(codes=FAKE + 16), dlc.DLC_ERR_ALIGNMENT),
    (lambda: quantize(spec=((32, 0, 4096),)), dlc.DLC_ERR_ALIGNMENT),
    (lambda: quantize(stride=4000), dlc.DLC_ERR_ALIGNMENT),
    (lambda: quantize(spec=((0, 0, 0),)), dlc.DLC_ERR_INVALID_ARGUMENT),
    (lambda: quantize(spec=((0, 0, 4097),)), dlc.DLC_ERR_INVALID_ARGUMENT),
    (lambda: quantize(spec=((0, 0, 1 << 32),), stride=1 << 33), dlc.DLC_ERR_INVALID_ARGUMENT),
    (lambda: quantize(spec=((1 << 38, 0, 64),)), dlc.DLC_ERR_INVALID_ARGUMENT),
    (lambda: quantize(spec=((0, 0, 128), (64, 128, 64)), stride=4096), dlc.DLC_ERR_INVALID_ARGUMENT),
    (lambda: quantize(spec=((0, 0, 128), (128, 64, 64)), stride=4096), dlc.DLC_ERR_INVALID_ARGUMENT),
    (lambda: quantize(present=[0, 0]), dlc.DLC_ERR_NO_QUORUM),
    (lambda: quantize(ws_bytes=16), dlc.DLC_ERR_WORKSPACE),
    (lambda: quantize(ws=None), dlc.DLC_ERR_WORKSPACE),
    (lambda: quantize(flags=16), dlc.DLC_ERR_INVALID_ARGUMENT),
    (lambda: quantize(flags=dlc.DLC_DEBUG_CHECKS | dlc.DLC_RANGE_GIVEN), dlc.DLC_ERR_INVALID_ARGUMENT),
    (lambda: merge(weights=(0.0, 0.0)), dlc.DLC_ERR_NO_QUORUM),
    (lambda: merge(weights=(1.0, -1.0)), dlc.DLC_ERR_INVALID_ARGUMENT),
    (lambda: merge(weights=(1.0, float("nan"))), dlc.DLC_ERR_INVALID_ARGUMENT),
    (lambda: merge(weights=(1.0, float("inf"))), dlc.DLC_ERR_INVALID_ARGUMENT),
    (lambda: merge(lr=float("nan")), dlc.DLC_ERR_INVALID_ARGUMENT),
    (lambda: merge(flags=1), dlc.DLC_ERR_INVALID_ARGUMENT),
    (lambda: merge(theta=FAKE + 8), dlc.DLC_ERR_ALIGNMENT),
    (lambda: merge(k=0, weights=()), dlc.DLC_ERR_INVALID_ARGUMENT),
    (lambda: quantize_bases(bases=None), dlc.DLC_ERR_INVALID_ARGUMENT),
    (lambda: quantize_bases(bases=(FAKE, 0)), dlc.DLC_ERR_INVALID_ARGUMENT),
    (lambda: quantize_bases(bases=(FAKE, 0), present=(1, 0)), dlc.DLC_ERR_WORKSPACE),
    (lambda: quantize_bases(present=(0, 0)), dlc.DLC_ERR_NO_QUORUM),
    (lambda: quantize_bases(bases=(FAKE + 8, FAKE)), dlc.DLC_ERR_ALIGNMENT),
    (lambda: broadcast(k=0), dlc.DLC_ERR_INVALID_ARGUMENT),
    (lambda: broadcast(theta=None), dlc.DLC_ERR_INVALID_ARGUMENT),
    (lambda: broadcast(theta=FAKE + 4), dlc.DLC_ERR_ALIGNMENT),
    (lambda: broadcast(stride=100), dlc.DLC_ERR_ALIGNMENT),
    (lambda: broadcast(spec=((0, 0, 0),)), dlc.DLC_ERR_INVALID_ARGUMENT),
    (lambda: cycle_ws(first=(1, 1)), dlc.DLC_ERR_INVALID_ARGUMENT),
    (lambda: cycle_ws(first=(0, 1, 0)), dlc.DLC_ERR_INVALID_ARGUMENT),
    (lambda: cycle_ws(first=(0, 0, 0)), dlc.DLC_ERR_INVALID_ARGUMENT),
    (lambda: cycle_ws(first=(0,)), dlc.DLC_ERR_INVALID_ARGUMENT),
    (lambda: cycle(flags=8), dlc.DLC_ERR_INVALID_ARGUMENT),
    (lambda: cycle(flags=4, ws_bytes=64), dlc.DLC_ERR_WORKSPACE),
    (lambda: cycle(weights=((1.0, 1.0), (0.0, 0.0))), dlc.DLC_ERR_NO_QUORUM),
    (lambda: cycle(weights=((1.0, 1.0), (1.0, -2.0))), dlc.DLC_ERR_INVALID_ARGUMENT),
    (lambda: cycle(ws_bytes=64), dlc.DLC_ERR_WORKSPACE),
    (lambda: cycle(codes=FAKE + 32), dlc.DLC_ERR_ALIGNMENT),
    (lambda: cycle(first=(0, 2, 1)), dlc.DLC_ERR_INVALID_ARGUMENT),
    (lambda: cycle(spec=((0, 0, 4096), (0, 4096, 64))), dlc.DLC_ERR_INVALID_ARGUMENT),
    (lambda: cycle_lanes(n_lanes=0), dlc.DLC_ERR_INVALID_ARGUMENT),
    (lambda: cycle_lanes(n_lanes=9), dlc.DLC_ERR_INVALID_ARGUMENT),
    (lambda: cycle_lanes(streams=False), dlc.DLC_ERR_INVALID_ARGUMENT),
    (lambda: cycle_lanes(flags=4), dlc.DLC_ERR_INVALID_ARGUMENT),
    (lambda: cycle_lanes(weights=((1.0, 1.0), (0.0, 0.0))), dlc.DLC_ERR_NO_QUORUM),
    (lambda: cycle_lanes(ws_bytes=64), dlc.DLC_ERR_WORKSPACE),
    (lambda: lanes_ws_short(), dlc.DLC_ERR_WORKSPACE),
    (lambda: quantize_static(**BIG_STATIC), dlc.DLC_ERR_WORKSPACE),
    (lambda: quantize_static(**BIG_STATIC, present=[1] * 15 + [0]), dlc.DLC_ERR_WORKSPACE),
    (lambda: quantize_static(k=65), dlc.DLC_ERR_INVALID_ARGUMENT),
    (lambda: quantize_static(flags=16), dlc.DLC_ERR_INVALID_ARGUMENT),
    (lambda: quantize_static(flags=dlc.DLC_DEBUG_CHECKS | dlc.DLC_RANGE_GIVEN), dlc.DLC_ERR_INVALID_ARGUMENT),
    (lambda: quantize_static(spec=((0, 0, 4097),)), dlc.DLC_ERR_INVALID_ARGUMENT),
    (lambda: quantize_static(present=[0, 0]), dlc.DLC_ERR_NO_QUORUM),
])
def test_argument_errors(call, code):
    assert call() == code
    assert dlc.dlc_last_error() != ""


def test_the_package_fails_loudly_without_its_library(tmp_path):
    """A copy of the package without libdlc.so must refuse to import (no fallback)."""
    import shutil
    import subprocess
    import sys
    src = os.path.join(ROOT, "diloco_outer_step_amd")
    dst = tmp_path / "diloco_outer_step_amd"
    shutil.copytree(src, dst, ignore=shutil.ignore_patterns("*.so", "__pycache__", "csrc"))
    r = subprocess.run([sys.executable, "-c", "import diloco_outer_step_amd"], cwd=tmp_path, capture_output=True,
                       text=True, timeout=300)
    assert r.returncode != 0 and "libdlc.so is missing" in r.stderr


def test_the_product_path_never_touches_the_oracle():
    """Neither the package nor the native sources import, load or name the CPU oracle."""
    pkg = os.path.join(ROOT, "diloco_outer_step_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f), encoding="utf-8").read()
                assert not re.search(r"\boracle\b", text), os.path.join(dirpath, f)


def test_static_scratch_limit_matches_the_workspace_sizes():
    """The static-scratch call takes exactly the calls whose workspace fits it."""
    assert dlc.DLC_STATIC_SCRATCH_BYTES == 64 << 20
    need = dlc.dlc_workspace_bytes(16, [(0, 0, 1 << 27)])
    assert need > dlc.DLC_STATIC_SCRATCH_BYTES
    assert "static scratch" in (quantize_static(**BIG_STATIC) and dlc.dlc_last_error())
    # the 135M set's largest fragment (its 28M-param embedding) at K = 4 fits
    assert dlc.dlc_workspace_bytes(4, [(0, 0, 49152 * 576)]) <= dlc.DLC_STATIC_SCRATCH_BYTES
