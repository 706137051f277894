"""dlc_quantize_static, the quantize call for callers that cannot allocate, against
dlc_quantize with a caller-allocated workspace: codes, codebooks and ranges bit
for bit (both run the same kernels; only the workspace differs), on calls in a
row that share the device's static scratch: a fragment of the 135M set (K = 4),
then a smaller ragged call (K = 3), then the first call again and the first
call with the oracle's ranges given."""
import pytest
import torch

import diloco_outer_step_amd as dlc
from tests import parity
from tests.test_gpu_parity import case_inputs

pytestmark = pytest.mark.gpu

DEV = "cuda"


def with_workspace(inp, given=None):
    k, stride = inp.theta_L.shape
    codes, cb, rng = dlc.outputs_for(k, stride, len(inp.tensors), DEV)
    if given is not None:
        rng.copy_(given)
    ws = dlc.alloc_workspace(k, inp.tensors, DEV)
    dlc.dlc_quantize(inp.theta_g, inp.theta_L, inp.tensors, codes, cb, rng, ws, present=inp.present,
                     range_given=given is not None)
    return codes, cb, rng


def static(inp, given=None):
    k, stride = inp.theta_L.shape
    codes, cb, rng = dlc.outputs_for(k, stride, len(inp.tensors), DEV)
    if given is not None:
        rng.copy_(given)
    dlc.dlc_quantize_static(inp.theta_g, inp.theta_L, inp.tensors, codes, cb, rng, present=inp.present,
                            range_given=given is not None)
    return codes, cb, rng


def assert_same(inp, a, b):
    torch.cuda.synchronize()
    for i, p in enumerate(inp.present):
        if not p:
            continue
        assert torch.equal(a[1][i], b[1][i]), f"codebook of learner {i}"
        assert torch.equal(a[2][i], b[2][i]), f"range of learner {i}"
        for (_, lo, n) in inp.tensors:
            assert torch.equal(a[0][i, lo:lo + n], b[0][i, lo:lo + n]), f"codes of learner {i}"


def test_static_scratch_matches_a_caller_workspace_on_calls_in_a_row():
    big = case_inputs("c2_median_fragment")
    small = case_inputs("ragged_k3")
    assert dlc.dlc_workspace_bytes(big.theta_L.shape[0], big.tensors) > \
        dlc.dlc_workspace_bytes(small.theta_L.shape[0], small.tensors)
    first = static(big)
    assert_same(big, first, with_workspace(big))
    print("[no-alloc] 135M-set fragment (K = 4) bit-identical", flush=True)
    second = static(small)
    assert_same(small, second, with_workspace(small))
    print("[no-alloc] smaller ragged call (K = 3) bit-identical", flush=True)
    again = static(big)
    assert_same(big, again, first)
    orc = parity.oracle_step(big)
    r, _ = parity.oracle_ranges_tensor(orc, big)
    assert_same(big, static(big, r.to(DEV)), with_workspace(big, r.to(DEV)))
    print("[no-alloc] repeated and pinned-range calls bit-identical", flush=True)


def test_static_scratch_on_a_capturing_stream():
    """The call under HIP graph capture (where allocation is not allowed), replayed
    several times with eager work between the replays: every replay equals the
    eager call."""
    inp = case_inputs("ragged_k3")
    k, stride = inp.theta_L.shape
    want = with_workspace(inp)
    codes, cb, rng = dlc.outputs_for(k, stride, len(inp.tensors), DEV)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        dlc.dlc_quantize_static(inp.theta_g, inp.theta_L, inp.tensors, codes, cb, rng, stream=s)  # warm-up
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        dlc.dlc_quantize_static(inp.theta_g, inp.theta_L, inp.tensors, codes, cb, rng, stream=s)
    for rep in range(3):
        codes.fill_(0)
        cb.fill_(0)
        rng.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert_same(inp, (codes, cb, rng), want)
        static(case_inputs("c2_median_fragment"))  # other work on the same scratch between replays
        torch.cuda.synchronize()
