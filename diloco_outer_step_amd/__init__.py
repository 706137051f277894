"""DiLoCo outer-step merge on one MI355X (gfx950): Python binding of libdlc.so.

The functions here carry the C ABI's names (include/dlc.h) and only marshal
arguments: torch tensors supply device memory, torch's current HIP stream is the
default stream, and every step of the computation runs in the library's kernels.
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
LIB_PATH = os.path.join(_PKG, "libdlc.so")

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

EXPORTED = (
    "dlc_fragment_plan", "dlc_workspace_bytes", "dlc_quantize_range", "dlc_quantize_encode",
    "dlc_quantize", "dlc_quantize_bases", "dlc_merge_outer_step", "dlc_merge_weights", "dlc_broadcast",
    "dlc_cycle_workspace_bytes", "dlc_outer_cycle", "dlc_outer_cycle_lanes", "dlc_ring_workspace_bytes", "dlc_ring_outer_step",
    "dlc_rda_workspace_bytes", "dlc_rda_outer_step", "dlc_last_error", "dlc_version",
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
        "dlc_merge_outer_step": [vp, vp, vp, i64, i32, vp, vp, tp, i32, ctypes.c_double,
                                 ctypes.c_double, u32, vp],
        "dlc_quantize_bases": [vp, vp, i64, i32, vp, tp, i32, vp, vp, vp, vp, sz, vp],
        "dlc_merge_weights": [i32, vp, vp, i32, ctypes.c_double, vp, vp],
        "dlc_broadcast": [vp, vp, i64, i32, vp, tp, i32, vp],
        "dlc_ring_workspace_bytes": [i32, tp, i32, ctypes.POINTER(sz)],
        "dlc_ring_outer_step": [vp, vp, vp, i64, i32, tp, i32, ctypes.c_double, ctypes.c_double, vp, vp, vp, vp,
                                vp, sz, vp],
        "dlc_rda_workspace_bytes": [i32, tp, i32, ctypes.POINTER(sz)],
        "dlc_rda_outer_step": [vp, vp, vp, i64, i32, tp, i32, vp, ctypes.c_double, ctypes.c_double, vp, vp, vp, vp,
                               vp, sz, vp],
        "dlc_cycle_workspace_bytes": [i32, tp, vp, i32, ctypes.POINTER(sz)],
        "dlc_outer_cycle": [vp, vp, vp, i64, i32, vp, tp, vp, i32, vp, vp, vp, ctypes.c_double, ctypes.c_double,
                            u32, vp, sz, vp, vp],
        "dlc_outer_cycle_lanes": [vp, vp, vp, i64, i32, vp, tp, vp, i32, vp, vp, vp, ctypes.c_double,
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


def _learner_stride(theta_L: torch.Tensor) -> int:
    if theta_L.dim() != 2 or not theta_L.is_contiguous():
        raise ValueError("theta_L must be a contiguous [K, learner_stride] tensor")
    return theta_L.shape[1]


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
    k = theta_L.shape[0]
    arr, n = _tensors(tensors)
    _buf, pres = _present(present, k)
    _check(_lib.dlc_quantize_range(_ptr(theta_g), _ptr(theta_L), _learner_stride(theta_L), k, pres, arr, n,
                                   _ptr(range_out), _ptr(workspace), workspace.numel(), _stream(stream)))


def dlc_quantize_encode(theta_g, theta_L, tensors, range_in, codes, codebook, workspace, present=None,
                        stream=None):
    k = theta_L.shape[0]
    arr, n = _tensors(tensors)
    _buf, pres = _present(present, k)
    _check(_lib.dlc_quantize_encode(_ptr(theta_g), _ptr(theta_L), _learner_stride(theta_L), k, pres, arr, n,
                                    _ptr(range_in), _ptr(codes), _ptr(codebook), _ptr(workspace),
                                    workspace.numel(), _stream(stream)))


def dlc_quantize(theta_g, theta_L, tensors, codes, codebook, range_io, workspace, present=None,
                 range_given=False, stream=None, debug_checks=False):
    """debug_checks: raise DlcError (code DLC_ERR_NON_FINITE) when a present learner's
    pseudo-gradient holds NaN or Inf; the call then synchronizes the stream."""
    k = theta_L.shape[0]
    arr, n = _tensors(tensors)
    _buf, pres = _present(present, k)
    flags = (DLC_RANGE_GIVEN if range_given else 0) | (DLC_DEBUG_CHECKS if debug_checks else 0)
    _check(_lib.dlc_quantize(_ptr(theta_g), _ptr(theta_L), _learner_stride(theta_L), k, pres, arr, n,
                             _ptr(codes), _ptr(codebook), _ptr(range_io), flags, _ptr(workspace),
                             workspace.numel(), _stream(stream)))


def dlc_merge_outer_step(theta_g, momentum, codes, codebook, weights, tensors, lr=0.7, beta=0.9,
                         stream=None):
    k = codes.shape[0]
    if codes.dim() != 2 or not codes.is_contiguous():
        raise ValueError("codes must be a contiguous [K, learner_stride] uint8 tensor")
    w = (ctypes.c_double * k)(*[float(x) for x in weights])
    arr, n = _tensors(tensors)
    _check(_lib.dlc_merge_outer_step(_ptr(theta_g), _ptr(momentum), _ptr(codes), codes.shape[1], k,
                                     _ptr(codebook), ctypes.cast(w, ctypes.c_void_p), arr, n, float(lr),
                                     float(beta), 0, _stream(stream)))


def dlc_quantize_bases(bases, theta_L, tensors, codes, codebook, range_out, workspace, present=None,
                       stream=None):
    """dlc_quantize with learner i's pseudo-gradient taken against bases[i] (a
    device tensor laid out like theta_g)."""
    k = theta_L.shape[0]
    if len(bases) != k:
        raise ValueError("one base per learner")
    arr, n = _tensors(tensors)
    _buf, pres = _present(present, k)
    ptrs = (ctypes.c_void_p * k)(*[b.data_ptr() for b in bases])
    _check(_lib.dlc_quantize_bases(ctypes.cast(ptrs, ctypes.c_void_p), _ptr(theta_L), _learner_stride(theta_L), k,
                                   pres, arr, n, _ptr(codes), _ptr(codebook), _ptr(range_out), _ptr(workspace),
                                   workspace.numel(), _stream(stream)))


def dlc_merge_weights(tokens, arrival, quorum: int, grace: float):
    """-> (weights list, merge_time); raises NoQuorumError when the quorum is not met."""
    k = len(tokens)
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
    k = theta_L.shape[0]
    arr, n = _tensors(tensors)
    _check(_lib.dlc_ring_outer_step(_ptr(theta_g), _ptr(momentum), _ptr(theta_L), _learner_stride(theta_L), k, arr, n,
                                    float(lr), float(beta), _ptr(accum), _ptr(codes), _ptr(codebook), _ptr(range_out),
                                    _ptr(workspace), workspace.numel(), _stream(stream)))


def dlc_rda_workspace_bytes(n_learners: int, tensors) -> int:
    arr, n = _tensors(tensors)
    out = ctypes.c_size_t(0)
    _check(_lib.dlc_rda_workspace_bytes(int(n_learners), arr, n, ctypes.byref(out)))
    return out.value


def dlc_rda_outer_step(theta_g, momentum, theta_L, tensors, weights, codes, codebook, range_out, sq_norms, workspace,
                       lr=0.7, beta=0.9, stream=None):
    """One outer step merged by Radial-Directional Averaging; sq_norms is a device
    fp64 [K, n_tensors] output (squared norms of the dequantized pseudo-gradients)."""
    k = theta_L.shape[0]
    if sq_norms.dtype != torch.float64:
        raise ValueError("sq_norms must be float64")
    w = (ctypes.c_double * k)(*[float(x) for x in weights])
    arr, n = _tensors(tensors)
    _check(_lib.dlc_rda_outer_step(_ptr(theta_g), _ptr(momentum), _ptr(theta_L), _learner_stride(theta_L), k, arr, n,
                                   ctypes.cast(w, ctypes.c_void_p), float(lr), float(beta), _ptr(codes),
                                   _ptr(codebook), _ptr(range_out), _ptr(sq_norms), _ptr(workspace),
                                   workspace.numel(), _stream(stream)))


def dlc_broadcast(theta_g, theta_L, tensors, rows=None, stream=None):
    """Copy each tensor's theta_g into the learner rows of theta_L (all rows, or
    those with rows[i] true)."""
    k = theta_L.shape[0]
    arr, n = _tensors(tensors)
    _buf, sel = _present(rows, k)
    _check(_lib.dlc_broadcast(_ptr(theta_g), _ptr(theta_L), _learner_stride(theta_L), k, sel, arr, n,
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
    k = theta_L.shape[0]
    nf = len(fragment_first) - 1
    arr, _ = _tensors(tensors)
    _fb, fp = _fragments(fragment_first)
    w = (ctypes.c_double * (nf * k))(*[float(x) for row in weights for x in row])
    qs = _stream(quantize_stream)
    ms = qs if merge_stream is None else _stream(merge_stream)
    _check(_lib.dlc_outer_cycle(_ptr(theta_g), _ptr(momentum), _ptr(theta_L), _learner_stride(theta_L), k,
                                ctypes.cast(w, ctypes.c_void_p), arr, fp, nf, _ptr(codes), _ptr(codebook),
                                _ptr(range_out), float(lr), float(beta),
                                (DLC_BROADCAST if broadcast else 0) | (DLC_TWO_LANES if two_lanes else 0),
                                _ptr(workspace), workspace.numel(), qs, ms))


def dlc_outer_cycle_lanes(theta_g, momentum, theta_L, tensors, fragment_first, weights, codes, codebook, range_out,
                          workspace, streams, lr=0.7, beta=0.9, broadcast=False):
    """The fragment cycle with the non-empty fragments taking the given streams in
    turn (workspace of len(streams) times dlc_cycle_workspace_bytes)."""
    k = theta_L.shape[0]
    nf = len(fragment_first) - 1
    arr, _ = _tensors(tensors)
    _fb, fp = _fragments(fragment_first)
    w = (ctypes.c_double * (nf * k))(*[float(x) for row in weights for x in row])
    ss = (ctypes.c_void_p * max(1, len(streams)))(*[_stream(s).value for s in streams])
    _check(_lib.dlc_outer_cycle_lanes(_ptr(theta_g), _ptr(momentum), _ptr(theta_L), _learner_stride(theta_L), k,
                                      ctypes.cast(w, ctypes.c_void_p), arr, fp, nf, _ptr(codes), _ptr(codebook),
                                      _ptr(range_out), float(lr), float(beta), DLC_BROADCAST if broadcast else 0,
                                      _ptr(workspace), workspace.numel(), ctypes.cast(ss, ctypes.c_void_p),
                                      len(streams)))


def outputs_for(n_learners: int, learner_stride: int, n_tensors: int, device="cuda"):
    """Allocate (codes, codebook, range) buffers for a call."""
    codes = torch.empty((n_learners, learner_stride), dtype=torch.uint8, device=device)
    codebook = torch.empty((n_learners, n_tensors, DLC_N_BUCKETS), dtype=torch.float32, device=device)
    rng = torch.empty((n_learners, n_tensors, DLC_RANGE_FIELDS), dtype=torch.float32, device=device)
    return codes, codebook, rng
