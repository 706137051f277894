"""Guard bytes around and between the caller's buffers.

Every buffer a call touches (theta, momentum, codes, codebook, range, the
squared norms of Radial-Directional Averaging, the workspace) is allocated with
a 4 KB tail, and the buffer is filled with a sentinel before the call, so the
padding between tensors (offsets are rounded up to 64 elements), the rows and
entries of absent learners and the tails all hold it.  After each call:

  * every sentinel outside the elements the call may write is unchanged;
  * read-only inputs (theta_g for the quantize stage, the learner replicas,
    codes and codebooks for the merge) are unchanged everywhere;
  * the results inside the tensors are bit-identical to those of unguarded
    buffers (tests/parity.py's gpu_step).

A stray store past a buffer, into padding or into an absent learner's row would
change a sentinel; a stray load of padding into a result would change it from
the unguarded run's.
"""
import pytest
import torch

import diloco_outer_step_amd as dlc
from tests import parity
from tests.test_gpu_parity import case_inputs

pytestmark = pytest.mark.gpu

DEV = "cuda"
TAIL = 4096  # bytes after every buffer
SENT = dict(theta=1234.5, momentum=-4321.25, codebook=-7.75, range=-9.5, sq_norms=-3.25, codes=0xA5, workspace=0x5A)
CASES = ["ragged_k3", "many_tensors_k20", "max_learners_k64", "absent_k16_const"]


def guarded(shape, dtype, fill):
    """(whole buffer incl. tail, view of the requested shape at its start)."""
    n = 1
    for d in shape:
        n *= d
    extra = TAIL // torch.tensor([], dtype=dtype).element_size()
    buf = torch.full((n + extra,), fill, dtype=dtype, device=DEV)
    return buf, buf[:n].view(*shape)


def tensor_mask(length, tensors, which):
    """Boolean mask of the elements the tensors occupy (which = 0: offsets, 1: loffsets)."""
    m = torch.zeros(length, dtype=torch.bool, device=DEV)
    for t in tensors:
        m[t[which]:t[which] + t[2]] = True
    return m


def assert_sentinel(buf, view_numel, name, fill, inside=None):
    """The tail holds the sentinel, and so does every element of the view outside `inside`."""
    tail = buf[view_numel:]
    assert torch.all(tail == fill), f"{name}: {int((tail != fill).sum())} tail elements overwritten"
    if inside is not None:
        head = buf[:view_numel]
        bad = (head != fill) & ~inside
        assert not bad.any(), f"{name}: {int(bad.sum())} elements outside the tensors overwritten"


def guarded_call_buffers(inp):
    k, stride = inp.theta_L.shape
    t = len(inp.tensors)
    glen = inp.theta_g.numel()
    gmask = tensor_mask(glen, inp.tensors, 0)
    theta_buf, theta = guarded((glen,), torch.float32, SENT["theta"])
    mom_buf, mom = guarded((glen,), torch.float32, SENT["momentum"])
    theta[gmask] = inp.theta_g[gmask]
    mom[gmask] = inp.momentum[gmask]
    codes_buf, codes = guarded((k, stride), torch.uint8, SENT["codes"])
    cb_buf, cb = guarded((k, t, dlc.DLC_N_BUCKETS), torch.float32, SENT["codebook"])
    rng_buf, rng = guarded((k, t, dlc.DLC_RANGE_FIELDS), torch.float32, SENT["range"])
    return dict(gmask=gmask, theta=(theta_buf, theta), momentum=(mom_buf, mom), codes=(codes_buf, codes),
                codebook=(cb_buf, cb), range=(rng_buf, rng))


def check_quantize_outputs(b, inp):
    k, stride = inp.theta_L.shape
    t = len(inp.tensors)
    lmask = tensor_mask(stride, inp.tensors, 1)
    codes_inside = torch.zeros((k, stride), dtype=torch.bool, device=DEV)
    rows_inside = torch.zeros((k, t), dtype=torch.bool, device=DEV)
    for i, p in enumerate(inp.present):
        if p:
            codes_inside[i] = lmask
            rows_inside[i] = True
    assert_sentinel(b["codes"][0], k * stride, "codes", SENT["codes"], codes_inside.flatten())
    cb_inside = rows_inside[:, :, None].expand(k, t, dlc.DLC_N_BUCKETS).flatten()
    assert_sentinel(b["codebook"][0], cb_inside.numel(), "codebook", SENT["codebook"], cb_inside)
    rg_inside = rows_inside[:, :, None].expand(k, t, dlc.DLC_RANGE_FIELDS).flatten()
    assert_sentinel(b["range"][0], rg_inside.numel(), "range", SENT["range"], rg_inside)
    return rows_inside


@pytest.mark.parametrize("name", CASES)
def test_star_step_writes_only_inside_its_buffers(name):
    inp = case_inputs(name)
    k, stride = inp.theta_L.shape
    ref = parity.gpu_step(inp)
    b = guarded_call_buffers(inp)
    theta_buf, theta = b["theta"]
    mom_buf, mom = b["momentum"]
    codes, cb, rng = b["codes"][1], b["codebook"][1], b["range"][1]
    nws = max(256, dlc.dlc_workspace_bytes(k, inp.tensors))
    ws_buf, ws = guarded((nws,), torch.uint8, SENT["workspace"])
    theta_L0 = inp.theta_L.clone()
    theta0 = theta_buf.clone()
    dlc.dlc_quantize(theta, inp.theta_L, inp.tensors, codes, cb, rng, ws, present=inp.present)
    torch.cuda.synchronize()
    assert torch.equal(theta_buf, theta0), "the quantize stage wrote theta_g"
    assert torch.equal(inp.theta_L, theta_L0), "the quantize stage wrote the learner replicas"
    assert_sentinel(ws_buf, nws, "workspace", SENT["workspace"])
    check_quantize_outputs(b, inp)
    snap = {n: b[n][0].clone() for n in ("codes", "codebook", "range")}
    dlc.dlc_merge_outer_step(theta, mom, codes, cb, inp.weights, inp.tensors)
    torch.cuda.synchronize()
    for n in ("codes", "codebook", "range"):
        assert torch.equal(b[n][0], snap[n]), f"the merge wrote {n}"
    gmask = b["gmask"]
    assert_sentinel(theta_buf, theta.numel(), "theta", SENT["theta"], gmask)
    assert_sentinel(mom_buf, mom.numel(), "momentum", SENT["momentum"], gmask)
    # results inside the tensors: those of unguarded buffers, bit for bit
    assert torch.equal(theta[gmask], ref["theta"][gmask]) and torch.equal(mom[gmask], ref["momentum"][gmask])
    for i, p in enumerate(inp.present):
        if not p:
            continue
        assert torch.equal(cb[i], ref["codebook"][i]) and torch.equal(rng[i], ref["range"][i])
        for (_, lo, n) in inp.tensors:
            assert torch.equal(codes[i, lo:lo + n], ref["codes"][i, lo:lo + n])


@pytest.mark.parametrize("name", ["ragged_k3", "absent_k16_const", "max_learners_k64"])
def test_rda_step_writes_only_inside_its_buffers(name):
    inp = case_inputs(name)
    k, stride = inp.theta_L.shape
    t = len(inp.tensors)
    b = guarded_call_buffers(inp)
    theta_buf, theta = b["theta"]
    mom_buf, mom = b["momentum"]
    norms_buf, norms = guarded((k, t), torch.float64, SENT["sq_norms"])
    nws = max(256, dlc.dlc_rda_workspace_bytes(k, inp.tensors))
    ws_buf, ws = guarded((nws,), torch.uint8, SENT["workspace"])
    theta_L0 = inp.theta_L.clone()
    dlc.dlc_rda_outer_step(theta, mom, inp.theta_L, inp.tensors, inp.weights, b["codes"][1], b["codebook"][1],
                           b["range"][1], norms, ws)
    torch.cuda.synchronize()
    assert torch.equal(inp.theta_L, theta_L0), "the call wrote the learner replicas"
    rows_inside = check_quantize_outputs(b, inp)
    assert_sentinel(norms_buf, k * t, "sq_norms", SENT["sq_norms"], rows_inside.flatten())
    assert_sentinel(ws_buf, nws, "workspace", SENT["workspace"])
    assert_sentinel(theta_buf, theta.numel(), "theta", SENT["theta"], b["gmask"])
    assert_sentinel(mom_buf, mom.numel(), "momentum", SENT["momentum"], b["gmask"])


def test_ring_step_writes_only_inside_its_buffers():
    inp = case_inputs("ragged_k3")
    k, stride = inp.theta_L.shape
    t = len(inp.tensors)
    glen = inp.theta_g.numel()
    b = guarded_call_buffers(inp)
    theta_buf, theta = b["theta"]
    mom_buf, mom = b["momentum"]
    acc_buf, acc = guarded((k, stride), torch.float32, SENT["theta"])
    codes_buf, codes = guarded((k, stride), torch.uint8, SENT["codes"])
    cb_buf, cb = guarded((k * t, dlc.DLC_N_BUCKETS), torch.float32, SENT["codebook"])
    rng_buf, rng = guarded((k * t, dlc.DLC_RANGE_FIELDS), torch.float32, SENT["range"])
    nws = max(256, dlc.dlc_ring_workspace_bytes(k, inp.tensors))
    ws_buf, ws = guarded((nws,), torch.uint8, SENT["workspace"])
    dlc.dlc_ring_outer_step(theta, mom, inp.theta_L, inp.tensors, acc, codes, cb, rng, ws)
    torch.cuda.synchronize()
    lmask = tensor_mask(stride, inp.tensors, 1).repeat(k)
    assert_sentinel(acc_buf, k * stride, "accum", SENT["theta"], lmask)
    assert_sentinel(codes_buf, k * stride, "codes", SENT["codes"], lmask)
    assert_sentinel(cb_buf, cb.numel(), "codebook", SENT["codebook"])
    assert_sentinel(rng_buf, rng.numel(), "range", SENT["range"])
    assert_sentinel(ws_buf, nws, "workspace", SENT["workspace"])
    assert_sentinel(theta_buf, glen, "theta", SENT["theta"], b["gmask"])
    assert_sentinel(mom_buf, glen, "momentum", SENT["momentum"], b["gmask"])
