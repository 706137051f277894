"""dlc_quantize with DLC_DEBUG_CHECKS: a NaN or an infinity in a present learner's
pseudo-gradient is reported (DLC_ERR_NON_FINITE, naming the lowest (learner,
tensor) pair); such inputs are outside the contract, so the other pairs' outputs
are checked against a clean run, and the calls without the flag must stay within
their buffers and return normally."""
import pytest
import torch

import diloco_outer_step_amd as dlc
import workloads

pytestmark = pytest.mark.gpu

DEV = "cuda"
SIZES = [4096 * 3 + 5, 64 * 9, 100003]


def inputs(k=3):
    cfg = workloads.custom("debug", SIZES, k)
    return workloads.fragment_inputs(cfg, list(range(len(SIZES))), DEV)


def quantize(inp, theta_L, present=None, debug=False):
    k, stride = theta_L.shape
    codes, cb, rng = dlc.outputs_for(k, stride, len(inp.tensors), DEV)
    ws = dlc.alloc_workspace(k, inp.tensors, DEV)
    dlc.dlc_quantize(inp.theta_g, theta_L, inp.tensors, codes, cb, rng, ws, present=present, debug_checks=debug)
    torch.cuda.synchronize()
    return codes, cb, rng


def test_clean_inputs_pass_and_match_the_unchecked_call():
    inp = inputs()
    plain = quantize(inp, inp.theta_L)
    checked = quantize(inp, inp.theta_L, debug=True)
    for o, lo, n in inp.tensors:  # codes outside the tensors' ranges are never written
        assert torch.equal(plain[0][:, lo:lo + n], checked[0][:, lo:lo + n])
    assert torch.equal(plain[1], checked[1])
    assert torch.equal(plain[2], checked[2])


def test_non_finite_pseudo_gradients_are_reported():
    inp = inputs()
    theta_L = inp.theta_L.clone()
    _, lo0, _ = inp.tensors[0]
    _, lo2, n2 = inp.tensors[2]
    theta_L[2, lo0 + 7] = float("inf")       # learner 2, tensor 0
    theta_L[1, lo2 + n2 - 1] = float("nan")  # learner 1, tensor 2 (its last element, in the tail tile)
    with pytest.raises(dlc.DlcError) as err:
        quantize(inp, theta_L, debug=True)
    assert err.value.code == dlc.DLC_ERR_NON_FINITE
    assert "learner 1, tensor 2" in str(err.value)

    # without the flag the call returns normally; every clean (learner, tensor) pair
    # is unaffected by the others
    codes, cb, rng = quantize(inp, theta_L)
    ref_codes, ref_cb, ref_rng = quantize(inp, inp.theta_L)
    bad = {(2, 0), (1, 2)}
    for t, (o, lo, n) in enumerate(inp.tensors):
        for i in range(theta_L.shape[0]):
            if (i, t) in bad:
                # a pair with a NaN or an infinity: degenerate range, every code 0
                assert not torch.isfinite(rng[i, t, 0])
                assert int(codes[i, lo:lo + n].max()) == 0
                continue
            assert torch.equal(codes[i, lo:lo + n], ref_codes[i, lo:lo + n]), (i, t)
            assert torch.equal(cb[i, t], ref_cb[i, t]), (i, t)
            assert torch.equal(rng[i, t], ref_rng[i, t]), (i, t)


def test_an_absent_learner_is_not_checked():
    inp = inputs()
    theta_L = inp.theta_L.clone()
    theta_L[1, inp.tensors[0][1]] = float("nan")
    quantize(inp, theta_L, present=[1, 0, 1], debug=True)  # learner 1 is never read
    with pytest.raises(dlc.DlcError) as err:
        quantize(inp, theta_L, present=[1, 1, 1], debug=True)
    assert "learner 1, tensor 0" in str(err.value)
