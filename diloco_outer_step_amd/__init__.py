"""DiLoCo outer-step merge on one MI355X (gfx950): Python binding of libdlc.so.

The functions here carry the C ABI's names (include/dlc.h) and only marshal
arguments: torch tensors supply device memory, torch's current HIP stream is the
default stream, and every step of the computation runs in the library's kernels.
Before each call the binding checks the buffers it passes (dtype, contiguity,
extent against the tensor list, one device, a GPU) and the lengths of weight and
presence lists, so no caller mistake reaches a kernel as an out-of-bounds access.
Importing this package fails loudly if the library has not been built
(``python diloco_outer_step_amd/build.py``).
"""
from __future__ import annotations

import ctypes
import itertools
import os
from typing import Optional, Sequence, Tuple

import numpy as np
import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# DLC_LIBRARY selects another build of the same library (the host-sanitized one
# for host-only tests); the default is the in-tree libdlc.so.
LIB_PATH = os.environ.get("DLC_LIBRARY") or os.path.join(_PKG, "libdlc.so")

DLC_OK = 0
DLC_ERR_INVALID_ARGUMENT = -1
DLC_ERR_ALIGNMENT = -2
DLC_ERR_NO_QUORUM = -3
DLC_ERR_WORKSPACE = -4
DLC_ERR_HIP = -5
DLC_ERR_NON_FINITE = -6
DLC_RANGE_GIVEN = 1
DLC_BROADCAST = 2
DLC_TWO_LANES = 4
DLC_DEBUG_CHECKS = 8
DLC_MAX_LEARNERS = 64
DLC_MAX_LANES = 8
DLC_N_BUCKETS = 256
DLC_ALIGN_ELEMS = 64
DLC_RANGE_FIELDS = 4
DLC_STATIC_SCRATCH_BYTES = 64 << 20

EXPORTED = (
    "dlc_fragment_plan", "dlc_workspace_bytes", "dlc_quantize_range", "dlc_quantize_encode",
    "dlc_quantize", "dlc_quantize_static", "dlc_quantize_bases", "dlc_merge_outer_step", "dlc_merge_weights", "dlc_broadcast",
    "dlc_cycle_workspace_bytes", "dlc_outer_cycle", "dlc_outer_cycle_lanes", "dlc_ring_workspace_bytes", "dlc_ring_outer_step",
    "dlc_rda_workspace_bytes", "dlc_rda_outer_step", "dlc_cycle_rda_workspace_bytes", "dlc_outer_cycle_rda",
    "dlc_last_error", "dlc_version",
)


class DlcError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"dlc error {code}: {message}")
        self.code = code


class NoQuorumError(DlcError):
    pass


class _Tensor(ctypes.Structure):
    _fields_ = [("offset", ctypes.c_int64), ("loffset", ctypes.c_int64), ("numel", ctypes.c_int64)]


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python diloco_outer_step_amd/build.py`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, u32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32, ctypes.c_size_t
    tp = ctypes.POINTER(_Tensor)
    sig = {
        "dlc_fragment_plan": [vp, i32, i32, vp, vp],
        "dlc_workspace_bytes": [i32, tp, i32, ctypes.POINTER(sz)],
        "dlc_quantize_range": [vp, vp, i64, i32, vp, tp, i32, vp, vp, sz, vp],
        "dlc_quantize_encode": [vp, vp, i64, i32, vp, tp, i32, vp, vp, vp, vp, sz, vp],
        "dlc_quantize": [vp, vp, i64, i32, vp, tp, i32, vp, vp, vp, u32, vp, sz, vp],
        "dlc_quantize_static": [vp, vp, i64, i32, vp, tp, i32, vp, vp, vp, u32, vp],
        "dlc_merge_outer_step": [vp, vp, vp, i64, i32, vp, vp, tp, i32, ctypes.c_double,
                                 ctypes.c_double, u32, vp],
        "dlc_quantize_bases": [vp, vp, i64, i32, vp, tp, i32, vp, vp, vp, vp, sz, vp],
        "dlc_merge_weights": [i32, vp, vp, i32, ctypes.c_double, vp, vp],
        "dlc_broadcast": [vp, vp, i64, i32, vp, tp, i32, vp],
        "dlc_ring_workspace_bytes": [i32, tp, i32, ctypes.POINTER(sz)],
        "dlc_ring_outer_step": [vp, vp, vp, i64, i32, tp, i32, ctypes.c_double, ctypes.c_double, vp, vp, vp, vp,
                                vp, sz, vp],
        "dlc_rda_workspace_bytes": [i32, tp, i32, ctypes.POINTER(sz)],
        "dlc_rda_outer_step": [vp, vp, vp, vp, i64, i32, tp, i32, vp, ctypes.c_double, ctypes.c_double, vp, vp, vp,
                               vp, vp, sz, vp],
        "dlc_cycle_workspace_bytes": [i32, tp, vp, i32, ctypes.POINTER(sz)],
        "dlc_outer_cycle": [vp, vp, vp, i64, i32, vp, tp, vp, i32, vp, vp, vp, ctypes.c_double, ctypes.c_double,
                            u32, vp, sz, vp, vp],
        "dlc_outer_cycle_lanes": [vp, vp, vp, i64, i32, vp, tp, vp, i32, vp, vp, vp, ctypes.c_double,
                                  ctypes.c_double, u32, vp, sz, vp, i32],
        "dlc_cycle_rda_workspace_bytes": [i32, tp, vp, i32, ctypes.POINTER(sz)],
        "dlc_outer_cycle_rda": [vp, vp, vp, i64, i32, vp, tp, vp, i32, vp, vp, vp, vp, ctypes.c_double,
                                ctypes.c_double, u32, vp, sz, vp, i32],
    }
    for name, args in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = i32
    for name in ("dlc_last_error", "dlc_version"):
        fn = getattr(lib, name)
        fn.argtypes = []
        fn.restype = ctypes.c_char_p
    return lib


_lib = _load()


def _check(rc: int) -> None:
    if rc != DLC_OK:
        msg = _lib.dlc_last_error().decode()
        if rc == DLC_ERR_NO_QUORUM:
            raise NoQuorumError(rc, msg)
        raise DlcError(rc, msg)


def _tensors(tensors: Sequence[Tuple[int, int, int]]):
    """dlc_tensor array of (offset, loffset, numel) triples: one int64 [n][3] array
    viewed as the C structs (the ctypes array keeps that buffer alive)."""
    n = len(tensors)
    if n == 0:
        return (_Tensor * 1)(), 0
    a = np.fromiter(itertools.chain.from_iterable(tensors), dtype=np.int64, count=3 * n)
    return (_Tensor * n).from_buffer(a), n


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


class _Checks:
    """Refuse buffers the C ABI would reach out of bounds or misread: wrong type,
    dtype, layout or size, then (after every other check, so that each of those
    can be exercised on host tensors) a buffer not on the call's device."""

    def __init__(self):
        self.bufs = []

    def need(self, t, name: str, dtype: torch.dtype, min_numel: int = 0):
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch.Tensor, not {type(t).__name__}")
        if t.dtype != dtype:
            raise ValueError(f"{name} must be {dtype}, not {t.dtype}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if t.numel() < min_numel:
            raise ValueError(f"{name} holds {t.numel()} elements; the call needs at least {min_numel}")
        self.bufs.append((name, t))

    def learners(self, theta_L, tensors, name: str = "theta_L") -> Tuple[int, int]:
        """(K, learner_stride) of a [K, learner_stride] fp32 tensor whose rows hold
        every tensor's [loffset, loffset + numel)."""
        if not isinstance(theta_L, torch.Tensor) or theta_L.dim() != 2:
            raise ValueError(f"{name} must be a [K, learner_stride] tensor")
        self.need(theta_L, name, torch.float32)
        if _extents(tensors)[1] > theta_L.shape[1]:
            raise ValueError(f"a tensor reaches past {name}'s row length {theta_L.shape[1]}")
        return theta_L.shape[0], theta_L.shape[1]

    def rows(self, t, name: str, k: int, stride: int, dtype: torch.dtype):
        """A [k, stride] buffer mirroring the learner rows (codes, accumulators)."""
        self.need(t, name, dtype)
        if tuple(t.shape) != (k, stride):
            raise ValueError(f"{name} must have shape ({k}, {stride}), not {tuple(t.shape)}")

    def global_(self, tensors, **bufs):
        """theta_global-shaped fp32 buffers cover every tensor's [offset, offset + numel)."""
        end, _ = _extents(tensors)
        for name, t in bufs.items():
            self.need(t, name, torch.float32, end)

    def outputs(self, k: int, rows: int, codes=None, stride=None, codebook=None, rng=None, sq_norms=None):
        if codes is not None:
            self.rows(codes, "codes", k, stride, torch.uint8)
        if codebook is not None:
            self.need(codebook, "codebook", torch.float32, k * rows * DLC_N_BUCKETS)
        if rng is not None:
            self.need(rng, "range", torch.float32, k * rows * DLC_RANGE_FIELDS)
        if sq_norms is not None:
            self.need(sq_norms, "sq_norms", torch.float64, k * rows)

    def workspace(self, ws):
        self.need(ws, "workspace", torch.uint8)

    def done(self):
        """Every buffer on one device, and that device a GPU."""
        dev = None
        for name, t in self.bufs:
            if not t.is_cuda:
                raise ValueError(f"{name} must be a device tensor, not on {t.device}")
            if dev is None:
                dev = t.device
            elif t.device != dev:
                raise ValueError(f"{name} is on {t.device}, the call's other buffers on {dev}")


def _extents(tensors) -> Tuple[int, int]:
    """(end of the last tensor in theta_global, end of the last in a learner row)."""
    if len(tensors) == 0:
        return 0, 0
    return max(int(o) + int(n) for o, _, n in tensors), max(int(lo) + int(n) for _, lo, n in tensors)


def _weights(weights, k: int, name: str = "weights"):
    if len(weights) != k:
        raise ValueError(f"{name} holds {len(weights)} values for {k} learners")
    return (ctypes.c_double * k)(*[float(x) for x in weights])


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _present(present, k):
    if present is None:
        return None, None
    buf = (ctypes.c_uint8 * k)(*[1 if p else 0 for p in present])
    return buf, ctypes.cast(buf, ctypes.c_void_p)


def _present_list(present, k):
    if present is not None and len(present) != k:
        raise ValueError(f"present holds {len(present)} values for {k} learners")


def dlc_version() -> str:
    return _lib.dlc_version().decode()


def dlc_last_error() -> str:
    return _lib.dlc_last_error().decode()


def dlc_fragment_plan(numel: Sequence[int], n_fragments: int):
    """Greedy bin-packing of whole tensors -> (fragment_of list, fragment_numel list)."""
    n = len(numel)
    src = (ctypes.c_int64 * max(1, n))(*[int(v) for v in numel])
    frag = (ctypes.c_int32 * max(1, n))()
    loads = (ctypes.c_int64 * max(1, n_fragments))()
    _check(_lib.dlc_fragment_plan(ctypes.cast(src, ctypes.c_void_p), n, int(n_fragments),
                                  ctypes.cast(frag, ctypes.c_void_p), ctypes.cast(loads, ctypes.c_void_p)))
    return list(frag[:n]), list(loads[:n_fragments])


def dlc_workspace_bytes(n_learners: int, tensors) -> int:
    arr, n = _tensors(tensors)
    out = ctypes.c_size_t(0)
    _check(_lib.dlc_workspace_bytes(int(n_learners), arr, n, ctypes.byref(out)))
    return out.value


def alloc_workspace(n_learners: int, tensors, device="cuda") -> torch.Tensor:
    nbytes = max(256, dlc_workspace_bytes(n_learners, tensors))
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def dlc_quantize_range(theta_g, theta_L, tensors, range_out, workspace, present=None, stream=None):
    c = _Checks()
    k, stride = c.learners(theta_L, tensors)
    _present_list(present, k)
    c.global_(tensors, theta_g=theta_g)
    c.outputs(k, len(tensors), rng=range_out)
    c.workspace(workspace)
    c.done()
    arr, n = _tensors(tensors)
    _buf, pres = _present(present, k)
    _check(_lib.dlc_quantize_range(_ptr(theta_g), _ptr(theta_L), stride, k, pres, arr, n,
                                   _ptr(range_out), _ptr(workspace), workspace.numel(), _stream(stream)))


def dlc_quantize_encode(theta_g, theta_L, tensors, range_in, codes, codebook, workspace, present=None,
                        stream=None):
    c = _Checks()
    k, stride = c.learners(theta_L, tensors)
    _present_list(present, k)
    c.global_(tensors, theta_g=theta_g)
    c.outputs(k, len(tensors), codes, stride, codebook, range_in)
    c.workspace(workspace)
    c.done()
    arr, n = _tensors(tensors)
    _buf, pres = _present(present, k)
    _check(_lib.dlc_quantize_encode(_ptr(theta_g), _ptr(theta_L), stride, k, pres, arr, n,
                                    _ptr(range_in), _ptr(codes), _ptr(codebook), _ptr(workspace),
                                    workspace.numel(), _stream(stream)))


def dlc_quantize(theta_g, theta_L, tensors, codes, codebook, range_io, workspace, present=None,
                 range_given=False, stream=None, debug_checks=False):
    """debug_checks: raise DlcError (code DLC_ERR_NON_FINITE) when a present learner's
    pseudo-gradient holds NaN or Inf; the call then synchronizes the stream."""
    c = _Checks()
    k, stride = c.learners(theta_L, tensors)
    _present_list(present, k)
    c.global_(tensors, theta_g=theta_g)
    c.outputs(k, len(tensors), codes, stride, codebook, range_io)
    c.workspace(workspace)
    c.done()
    arr, n = _tensors(tensors)
    _buf, pres = _present(present, k)
    flags = (DLC_RANGE_GIVEN if range_given else 0) | (DLC_DEBUG_CHECKS if debug_checks else 0)
    _check(_lib.dlc_quantize(_ptr(theta_g), _ptr(theta_L), stride, k, pres, arr, n,
                             _ptr(codes), _ptr(codebook), _ptr(range_io), flags, _ptr(workspace),
                             workspace.numel(), _stream(stream)))


def dlc_quantize_static(theta_g, theta_L, tensors, codes, codebook, range_io, present=None, range_given=False,
                        stream=None, debug_checks=False):
    """dlc_quantize with the library's static device scratch as its workspace (no
    workspace argument, nothing allocated): for callers that cannot allocate.
    Calls that overlap on one device race on the scratch."""
    c = _Checks()
    k, stride = c.learners(theta_L, tensors)
    _present_list(present, k)
    c.global_(tensors, theta_g=theta_g)
    c.outputs(k, len(tensors), codes, stride, codebook, range_io)
    c.done()
    arr, n = _tensors(tensors)
    _buf, pres = _present(present, k)
    flags = (DLC_RANGE_GIVEN if range_given else 0) | (DLC_DEBUG_CHECKS if debug_checks else 0)
    _check(_lib.dlc_quantize_static(_ptr(theta_g), _ptr(theta_L), stride, k, pres, arr, n, _ptr(codes),
                                    _ptr(codebook), _ptr(range_io), flags, _stream(stream)))


def dlc_merge_outer_step(theta_g, momentum, codes, codebook, weights, tensors, lr=0.7, beta=0.9,
                         stream=None):
    if not isinstance(codes, torch.Tensor) or codes.dim() != 2:
        raise ValueError("codes must be a [K, learner_stride] uint8 tensor")
    k, stride = codes.shape
    w = _weights(weights, k)
    c = _Checks()
    c.rows(codes, "codes", k, stride, torch.uint8)
    c.global_(tensors, theta_g=theta_g, momentum=momentum)
    if _extents(tensors)[1] > stride:
        raise ValueError(f"a tensor reaches past learner_stride {stride}")
    c.outputs(k, len(tensors), codebook=codebook)
    c.done()
    arr, n = _tensors(tensors)
    _check(_lib.dlc_merge_outer_step(_ptr(theta_g), _ptr(momentum), _ptr(codes), codes.shape[1], k,
                                     _ptr(codebook), ctypes.cast(w, ctypes.c_void_p), arr, n, float(lr),
                                     float(beta), 0, _stream(stream)))


def dlc_quantize_bases(bases, theta_L, tensors, codes, codebook, range_out, workspace, present=None,
                       stream=None):
    """dlc_quantize with learner i's pseudo-gradient taken against bases[i] (a
    device tensor laid out like theta_g; None for a learner that is not present)."""
    c = _Checks()
    k, stride = c.learners(theta_L, tensors)
    if len(bases) != k:
        raise ValueError("one base per learner")
    _present_list(present, k)
    c.global_(tensors, **{f"bases[{i}]": b for i, b in enumerate(bases) if present is None or present[i]})
    c.outputs(k, len(tensors), codes, stride, codebook, range_out)
    c.workspace(workspace)
    c.done()
    arr, n = _tensors(tensors)
    _buf, pres = _present(present, k)
    ptrs = (ctypes.c_void_p * k)(*[0 if b is None else b.data_ptr() for b in bases])
    _check(_lib.dlc_quantize_bases(ctypes.cast(ptrs, ctypes.c_void_p), _ptr(theta_L), stride, k,
                                   pres, arr, n, _ptr(codes), _ptr(codebook), _ptr(range_out), _ptr(workspace),
                                   workspace.numel(), _stream(stream)))


def dlc_merge_weights(tokens, arrival, quorum: int, grace: float):
    """-> (weights list, merge_time); raises NoQuorumError when the quorum is not met."""
    k = len(tokens)
    if len(arrival) != k:
        raise ValueError(f"arrival holds {len(arrival)} values for {k} learners")
    t = (ctypes.c_double * k)(*[float(x) for x in tokens])
    a = (ctypes.c_double * k)(*[float(x) for x in arrival])
    w = (ctypes.c_double * k)()
    mt = ctypes.c_double(0.0)
    _check(_lib.dlc_merge_weights(k, ctypes.cast(t, ctypes.c_void_p), ctypes.cast(a, ctypes.c_void_p), int(quorum),
                                  float(grace), ctypes.cast(w, ctypes.c_void_p), ctypes.cast(ctypes.byref(mt),
                                                                                          ctypes.c_void_p)))
    return list(w), mt.value


def dlc_ring_workspace_bytes(n_learners: int, tensors) -> int:
    arr, n = _tensors(tensors)
    out = ctypes.c_size_t(0)
    _check(_lib.dlc_ring_workspace_bytes(int(n_learners), arr, n, ctypes.byref(out)))
    return out.value


def ring_buffers(theta_L, n_tensors: int):
    """(accum, codes, codebook, range, workspace-size-less) buffers for dlc_ring_outer_step."""
    k, stride = theta_L.shape
    dev = theta_L.device
    accum = torch.empty((k, stride), dtype=torch.float32, device=dev)
    codes = torch.empty((k, stride), dtype=torch.uint8, device=dev)
    codebook = torch.empty((k * n_tensors, DLC_N_BUCKETS), dtype=torch.float32, device=dev)
    rng = torch.empty((k * n_tensors, DLC_RANGE_FIELDS), dtype=torch.float32, device=dev)
    return accum, codes, codebook, rng


def dlc_ring_outer_step(theta_g, momentum, theta_L, tensors, accum, codes, codebook, range_out, workspace, lr=0.7,
                        beta=0.9, stream=None):
    c = _Checks()
    k, stride = c.learners(theta_L, tensors)
    c.global_(tensors, theta_g=theta_g, momentum=momentum)
    c.rows(accum, "accum", k, stride, torch.float32)
    c.outputs(k, len(tensors), codes, stride, codebook, range_out)
    c.workspace(workspace)
    c.done()
    arr, n = _tensors(tensors)
    _check(_lib.dlc_ring_outer_step(_ptr(theta_g), _ptr(momentum), _ptr(theta_L), stride, k, arr, n,
                                    float(lr), float(beta), _ptr(accum), _ptr(codes), _ptr(codebook), _ptr(range_out),
                                    _ptr(workspace), workspace.numel(), _stream(stream)))


def dlc_rda_workspace_bytes(n_learners: int, tensors) -> int:
    arr, n = _tensors(tensors)
    out = ctypes.c_size_t(0)
    _check(_lib.dlc_rda_workspace_bytes(int(n_learners), arr, n, ctypes.byref(out)))
    return out.value


def dlc_rda_outer_step(theta_g, momentum, theta_L, tensors, weights, codes, codebook, range_out, sq_norms, workspace,
                       lr=0.7, beta=0.9, stream=None, bases=None):
    """One outer step merged by Radial-Directional Averaging; sq_norms is a device
    fp64 [K, n_tensors] output (squared norms of the dequantized pseudo-gradients).
    bases: None (every learner against theta_g) or one device tensor per learner,
    laid out like theta_g, that learner's pseudo-gradient is taken against (None
    for a learner of weight 0)."""
    c = _Checks()
    k, stride = c.learners(theta_L, tensors)
    w = _weights(weights, k)
    c.global_(tensors, theta_g=theta_g, momentum=momentum)
    ptrs = None
    if bases is not None:
        if len(bases) != k:
            raise ValueError("one base per learner")
        c.global_(tensors, **{f"bases[{i}]": b for i, b in enumerate(bases) if weights[i] > 0})
        ptrs = (ctypes.c_void_p * k)(*[0 if b is None else b.data_ptr() for b in bases])
    c.outputs(k, len(tensors), codes, stride, codebook, range_out, sq_norms)
    c.workspace(workspace)
    c.done()
    arr, n = _tensors(tensors)
    _check(_lib.dlc_rda_outer_step(_ptr(theta_g), _ptr(momentum), _ptr(theta_L),
                                   None if ptrs is None else ctypes.cast(ptrs, ctypes.c_void_p), stride, k, arr, n,
                                   ctypes.cast(w, ctypes.c_void_p), float(lr), float(beta), _ptr(codes),
                                   _ptr(codebook), _ptr(range_out), _ptr(sq_norms), _ptr(workspace),
                                   workspace.numel(), _stream(stream)))


def dlc_broadcast(theta_g, theta_L, tensors, rows=None, stream=None):
    """Copy each tensor's theta_g into the learner rows of theta_L (all rows, or
    those with rows[i] true)."""
    c = _Checks()
    k, stride = c.learners(theta_L, tensors)
    if rows is not None and len(rows) != k:
        raise ValueError(f"rows holds {len(rows)} values for {k} learners")
    c.global_(tensors, theta_g=theta_g)
    c.done()
    arr, n = _tensors(tensors)
    _buf, sel = _present(rows, k)
    _check(_lib.dlc_broadcast(_ptr(theta_g), _ptr(theta_L), stride, k, sel, arr, n,
                              _stream(stream)))


def _fragments(fragment_first: Sequence[int]):
    buf = (ctypes.c_int32 * len(fragment_first))(*[int(v) for v in fragment_first])
    return buf, ctypes.cast(buf, ctypes.c_void_p)


def group_by_fragment(tensors, fragment_of, n_fragments):
    """Tensors reordered fragment by fragment (stable) -> (tensors, fragment_first,
    order), where order[j] is the original index of the j-th tensor."""
    order = sorted(range(len(tensors)), key=lambda t: (fragment_of[t], t))
    first = [0] * (n_fragments + 1)
    for t in order:
        first[fragment_of[t] + 1] += 1
    for f in range(n_fragments):
        first[f + 1] += first[f]
    return [tensors[t] for t in order], first, order


def _cycle_checks(theta_g, momentum, theta_L, tensors, nf, weights, codes, codebook, range_out, workspace,
                  sq_norms=None):
    """Buffer checks of a fragment cycle -> (weights as a C array, K, learner_stride)."""
    c = _Checks()
    k, stride = c.learners(theta_L, tensors)
    if len(weights) != nf:
        raise ValueError(f"weights holds {len(weights)} rows for {nf} fragments")
    for f, row in enumerate(weights):
        if len(row) != k:
            raise ValueError(f"weights[{f}] holds {len(row)} values for {k} learners")
    c.global_(tensors, theta_g=theta_g, momentum=momentum)
    c.outputs(k, len(tensors), codes, stride, codebook, range_out, sq_norms)
    c.workspace(workspace)
    c.done()
    return (ctypes.c_double * (nf * k))(*[float(x) for row in weights for x in row]), k, stride


def dlc_cycle_workspace_bytes(n_learners: int, tensors, fragment_first) -> int:
    arr, _ = _tensors(tensors)
    _fb, fp = _fragments(fragment_first)
    out = ctypes.c_size_t(0)
    _check(_lib.dlc_cycle_workspace_bytes(int(n_learners), arr, fp, len(fragment_first) - 1, ctypes.byref(out)))
    return out.value


def dlc_outer_cycle(theta_g, momentum, theta_L, tensors, fragment_first, weights, codes, codebook, range_out,
                    workspace, lr=0.7, beta=0.9, broadcast=False, quantize_stream=None, merge_stream=None,
                    two_lanes=False):
    """One outer step over every fragment; weights is [n_fragments][n_learners].
    two_lanes: fragments alternate between the two streams (workspace of twice
    dlc_cycle_workspace_bytes)."""
    nf = len(fragment_first) - 1
    w, k, stride = _cycle_checks(theta_g, momentum, theta_L, tensors, nf, weights, codes, codebook, range_out, workspace)
    arr, _ = _tensors(tensors)
    _fb, fp = _fragments(fragment_first)
    qs = _stream(quantize_stream)
    ms = qs if merge_stream is None else _stream(merge_stream)
    _check(_lib.dlc_outer_cycle(_ptr(theta_g), _ptr(momentum), _ptr(theta_L), stride, k,
                                ctypes.cast(w, ctypes.c_void_p), arr, fp, nf, _ptr(codes), _ptr(codebook),
                                _ptr(range_out), float(lr), float(beta),
                                (DLC_BROADCAST if broadcast else 0) | (DLC_TWO_LANES if two_lanes else 0),
                                _ptr(workspace), workspace.numel(), qs, ms))


def dlc_outer_cycle_lanes(theta_g, momentum, theta_L, tensors, fragment_first, weights, codes, codebook, range_out,
                          workspace, streams, lr=0.7, beta=0.9, broadcast=False):
    """The fragment cycle with the non-empty fragments taking the given streams in
    turn (workspace of len(streams) times dlc_cycle_workspace_bytes)."""
    nf = len(fragment_first) - 1
    w, k, stride = _cycle_checks(theta_g, momentum, theta_L, tensors, nf, weights, codes, codebook, range_out, workspace)
    arr, _ = _tensors(tensors)
    _fb, fp = _fragments(fragment_first)
    ss = (ctypes.c_void_p * max(1, len(streams)))(*[_stream(s).value for s in streams])
    _check(_lib.dlc_outer_cycle_lanes(_ptr(theta_g), _ptr(momentum), _ptr(theta_L), stride, k,
                                      ctypes.cast(w, ctypes.c_void_p), arr, fp, nf, _ptr(codes), _ptr(codebook),
                                      _ptr(range_out), float(lr), float(beta), DLC_BROADCAST if broadcast else 0,
                                      _ptr(workspace), workspace.numel(), ctypes.cast(ss, ctypes.c_void_p),
                                      len(streams)))


def dlc_cycle_rda_workspace_bytes(n_learners: int, tensors, fragment_first) -> int:
    arr, _ = _tensors(tensors)
    _fb, fp = _fragments(fragment_first)
    out = ctypes.c_size_t(0)
    _check(_lib.dlc_cycle_rda_workspace_bytes(int(n_learners), arr, fp, len(fragment_first) - 1, ctypes.byref(out)))
    return out.value


def dlc_outer_cycle_rda(theta_g, momentum, theta_L, tensors, fragment_first, weights, codes, codebook, range_out,
                        sq_norms, workspace, streams, lr=0.7, beta=0.9, broadcast=False):
    """The fragment cycle on the given streams with every fragment merged by
    Radial-Directional Averaging; sq_norms is fp64 [n_learners][n_tensors]
    (workspace of len(streams) times dlc_cycle_rda_workspace_bytes)."""
    if sq_norms is None:
        raise ValueError("sq_norms is required")
    nf = len(fragment_first) - 1
    w, k, stride = _cycle_checks(theta_g, momentum, theta_L, tensors, nf, weights, codes, codebook, range_out,
                                 workspace, sq_norms)
    arr, _ = _tensors(tensors)
    _fb, fp = _fragments(fragment_first)
    ss = (ctypes.c_void_p * max(1, len(streams)))(*[_stream(s).value for s in streams])
    _check(_lib.dlc_outer_cycle_rda(_ptr(theta_g), _ptr(momentum), _ptr(theta_L), stride, k,
                                    ctypes.cast(w, ctypes.c_void_p), arr, fp, nf, _ptr(codes), _ptr(codebook),
                                    _ptr(range_out), _ptr(sq_norms), float(lr), float(beta),
                                    DLC_BROADCAST if broadcast else 0, _ptr(workspace), workspace.numel(),
                                    ctypes.cast(ss, ctypes.c_void_p), len(streams)))


def outputs_for(n_learners: int, learner_stride: int, n_tensors: int, device="cuda"):
    """Allocate (codes, codebook, range) buffers for a call."""
    codes = torch.empty((n_learners, learner_stride), dtype=torch.uint8, device=device)
    codebook = torch.empty((n_learners, n_tensors, DLC_N_BUCKETS), dtype=torch.float32, device=device)
    rng = torch.empty((n_learners, n_tensors, DLC_RANGE_FIELDS), dtype=torch.float32, device=device)
    return codes, codebook, rng
