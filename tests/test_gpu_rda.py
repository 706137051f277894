"""GPU tests of the outer step merged by Radial-Directional Averaging
(dlc_rda_outer_step) against the CPU oracle's rda_merge.

* quantization: codes, codebooks and ranges with the parity bar of
  tests/parity.py (the call quantizes exactly as dlc_quantize);
* merge: the oracle's rda_merge and nesterov evaluated on the GPU's own codes
  and codebooks give theta and momentum within one fp32 ulp (both sides compute
  in fp64 and differ only in the order of fp64 rounding), and the squared norms
  within 1e-12 relative;
* end to end against the oracle's own quantization: every element whose codes
  all match is within the theta/momentum tolerance of tests/parity.py;
* degenerate cases: learners that did not move (zero norms: a pure momentum
  step), zero-variance tensors, absent learners, one learner (the star step),
  more than 16 learners (the run-time learner loop), a full-size parameter set;
* learners on older bases (one call with bases) against the oracle's step with
  the same bases, and theta_global passed as every base equal to no bases.
"""
import numpy as np
import pytest
import torch

import diloco_outer_step_amd as dlc
import oracle
import workloads
from tests import parity
from tests.test_gpu_parity import case_inputs
from tests.test_gpu_stale import stale_inputs

pytestmark = pytest.mark.gpu

DEV = "cuda"
LR, BETA = 0.7, 0.9


def packed(sizes):
    offs, pos = [], 0
    for n in sizes:
        offs.append(pos)
        pos += (n + 63) // 64 * 64
    return [(o, o, n) for o, n in zip(offs, sizes)], pos


def rda_buffers(k, stride, n_tensors, tensors):
    codes, cb, rng = dlc.outputs_for(k, stride, n_tensors, DEV)
    norms = torch.zeros((k, n_tensors), dtype=torch.float64, device=DEV)
    ws = torch.empty(max(256, dlc.dlc_rda_workspace_bytes(k, tensors)), dtype=torch.uint8, device=DEV)
    return codes, cb, rng, norms, ws


def gpu_rda(inp):
    k, stride = inp.theta_L.shape
    codes, cb, rng, norms, ws = rda_buffers(k, stride, len(inp.tensors), inp.tensors)
    th, mo = inp.theta_g.clone(), inp.momentum.clone()
    dlc.dlc_rda_outer_step(th, mo, inp.theta_L, inp.tensors, inp.weights, codes, cb, rng, norms, ws, LR, BETA)
    torch.cuda.synchronize()
    return dict(codes=codes, codebook=cb, range=rng, sq_norms=norms, theta=th, momentum=mo)


def check_merge_on_gpu_codes(gpu, inp, theta0, mom0):
    """The oracle's RDA merge + Nesterov on the GPU's own quantized data."""
    w_hat = oracle.normalize_weights(inp.weights)
    codes, cb = parity.host(gpu["codes"]), parity.host(gpu["codebook"])
    norms = parity.host(gpu["sq_norms"])
    th_g, mo_g = parity.host(gpu["theta"]), parity.host(gpu["momentum"])
    exact = total = 0
    for t, (off, loff, n) in enumerate(inp.tensors):
        present = [i for i, w in enumerate(inp.weights) if w > 0]
        cs = [codes[i, loff:loff + n] for i in present]
        cbs = [cb[i, t] for i in present]
        for i, c, b in zip(present, cs, cbs):
            x = oracle.dequantize(c, b).astype(np.float64)
            want = float(np.sum(x * x))
            assert abs(norms[i, t] - want) <= 1e-12 * want + 1e-300, (i, t, norms[i, t], want)
        g = oracle.rda_merge(cs, cbs, [w_hat[i] for i in present])
        th_o, mo_o = oracle.nesterov(theta0[off:off + n], mom0[off:off + n], g, LR, BETA)
        d_th = parity.ulp_distance(th_g[off:off + n], th_o)
        d_mo = parity.ulp_distance(mo_g[off:off + n], mo_o)
        assert d_th.max() <= 1 and d_mo.max() <= 1, (t, int(d_th.max()), int(d_mo.max()))
        exact += int(np.sum(d_th == 0)) + int(np.sum(d_mo == 0))
        total += 2 * n
    assert exact >= 0.999 * total, f"{exact} of {total} bit-identical"


def make_inputs(seed, k, sizes, weights, unmoved=(), constant=()):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    tensors, stride = packed(sizes)
    theta = torch.randn(stride, generator=g, device=DEV) * 0.02
    for _, t in constant:  # exactly representable, so the constant move is exact
        off, _, n = tensors[t]
        theta[off:off + n] = 0.5
    mom = torch.randn(stride, generator=g, device=DEV) * 1e-3
    scales = torch.rand(k, generator=g, device=DEV) * 2e-3 + 2e-4
    theta_L = torch.stack([theta - torch.randn(stride, generator=g, device=DEV) * scales[i] for i in range(k)])
    for i in unmoved:
        theta_L[i] = theta
    for i, t in constant:  # learner i moved tensor t by exactly 2^-12: zero variance, nonzero mean
        off, loff, n = tensors[t]
        theta_L[i, loff:loff + n] = 0.5 - 2.0 ** -12
    present = [1 if w > 0 else 0 for w in weights]
    return workloads.StepInputs(theta, mom, theta_L.contiguous(), tensors, list(weights), present,
                                list(range(len(tensors))), stride)


SIZES = [1, 63, 65, 5000, 4096 * 3 + 1, 64 * 300 + 9, 100003]


@pytest.mark.parametrize("k", [1, 3, 8, 16, 20, 64])
def test_rda_against_oracle(k):
    rng = np.random.default_rng(k)
    w = [float(x) for x in rng.uniform(0.5, 3.0, k)]
    if k >= 3:
        w[1] = 0.0  # absent
    unmoved = (2,) if k >= 8 else ()
    constant = ((0, 3),) if k >= 3 else ()
    inp = make_inputs(20 + k, k, SIZES, w, unmoved, constant)
    gpu = gpu_rda(inp)
    theta0, mom0 = parity.host(inp.theta_g), parity.host(inp.momentum)
    check_merge_on_gpu_codes(gpu, inp, theta0, mom0)
    orc = oracle.outer_step(theta0, mom0, parity.host(inp.theta_L), inp.theta_L.shape[1], inp.tensors, inp.weights,
                            inp.present, LR, BETA, rule="rda")
    rep = parity.compare(gpu, orc, inp, pinned=False, state=False)
    if rep["flips"] == 0:
        for off, _, n in inp.tensors:
            th_o, th_g = orc["theta"][off:off + n], parity.host(gpu["theta"])[off:off + n]
            assert np.all(np.abs(th_g.astype(np.float64) - th_o) <= parity.ATOL + parity.RTOL * np.abs(th_o))
    for i, t in constant:
        n = inp.tensors[t][2]
        assert float(gpu["sq_norms"][i, t]) == n * 2.0 ** -24
    # absent learners' rows are untouched
    for i, wi in enumerate(w):
        if wi == 0:
            assert torch.all(gpu["sq_norms"][i] == 0)


def test_unmoved_learners_give_a_pure_momentum_step():
    k = 3
    inp = make_inputs(5, k, SIZES, [1.0, 2.0, 0.5], unmoved=(0, 1, 2))
    gpu = gpu_rda(inp)
    assert torch.all(gpu["sq_norms"] == 0)
    theta0, mom0 = parity.host(inp.theta_g), parity.host(inp.momentum)
    for off, _, n in inp.tensors:
        th_o, mo_o = oracle.nesterov(theta0[off:off + n], mom0[off:off + n], np.zeros(n), LR, BETA)
        np.testing.assert_array_equal(parity.host(gpu["theta"])[off:off + n], th_o)
        np.testing.assert_array_equal(parity.host(gpu["momentum"])[off:off + n], mo_o)


def test_one_learner_is_the_star_step():
    inp = make_inputs(6, 1, SIZES, [1.0])
    gpu = gpu_rda(inp)
    star = parity.gpu_step(inp, LR, BETA)
    for t, (_, loff, n) in enumerate(inp.tensors):  # the padding between tensors is never written
        assert torch.equal(gpu["codes"][:, loff:loff + n], star["codes"][:, loff:loff + n])
    assert torch.equal(gpu["codebook"], star["codebook"])
    d = parity.ulp_distance(parity.host(gpu["theta"]), parity.host(star["theta"]))
    assert d.max() <= 1 and np.mean(d == 0) >= 0.999


def test_identical_learners_are_the_star_step():
    k = 4
    inp = make_inputs(7, k, SIZES, [1.0, 2.0, 3.0, 4.0])
    inp.theta_L[:] = inp.theta_L[0].clone()
    gpu = gpu_rda(inp)
    star = parity.gpu_step(inp, LR, BETA)
    d = parity.ulp_distance(parity.host(gpu["theta"]), parity.host(star["theta"]))
    assert d.max() <= 2


def test_balanced_constant_learners_cancel():
    """Twelve learners move tensor 0 by constants, six up and six down, under equal
    weights: their directions cancel in real arithmetic, so g = 0 there and the
    step is the pure momentum step (the averaged direction left by rounding counts
    as zero); tensor 1 moves normally.  Tensor 0 has a size that is no power of
    two, so the norms round."""
    k, sizes = 12, [114687, 5000]
    inp = make_inputs(31, k, sizes, [1.0] * k)
    off, loff, n = inp.tensors[0]
    inp.theta_g[off:off + n] = 0.5
    rng = np.random.default_rng(31)
    signs = np.array([1.0] * 6 + [-1.0] * 6)
    rng.shuffle(signs)
    for i, c in enumerate(signs * 10.0 ** rng.uniform(-5, -3, k)):
        inp.theta_L[i, loff:loff + n] = float(np.float32(0.5) - np.float32(c))
    theta0, mom0 = parity.host(inp.theta_g), parity.host(inp.momentum)
    gpu = gpu_rda(inp)
    check_merge_on_gpu_codes(gpu, inp, theta0, mom0)
    th_o, mo_o = oracle.nesterov(theta0[off:off + n], mom0[off:off + n], np.zeros(n), LR, BETA)
    assert np.array_equal(parity.host(gpu["momentum"])[off:off + n], mo_o)
    assert np.array_equal(parity.host(gpu["theta"])[off:off + n], th_o)


def test_stale_bases_rda_against_oracle():
    """Learners that started from three versions of the global parameters (the
    digest's asynchronous learners), token weights, one learner absent, merged by
    Radial-Directional Averaging in one call: the quantization at the parity bar
    against the oracle's with the same bases, and the oracle's RDA merge and
    Nesterov step on the GPU's own codes within one ulp."""
    theta, mom, theta_L, tensors, bases = stale_inputs(5)
    k, stride = theta_L.shape
    weights = [4096.0 * (i + 1) for i in range(k)]
    weights[2] = 0.0
    present = [1 if w > 0 else 0 for w in weights]
    codes, cb, rng, norms, ws = rda_buffers(k, stride, len(tensors), tensors)
    th, mo = theta.clone(), mom.clone()
    passed = list(bases)
    passed[2] = None  # the absent learner needs no base
    dlc.dlc_rda_outer_step(th, mo, theta_L, tensors, weights, codes, cb, rng, norms, ws, LR, BETA, bases=passed)
    torch.cuda.synchronize()
    gpu = dict(codes=codes, codebook=cb, range=rng, sq_norms=norms, theta=th, momentum=mo)
    theta0, mom0 = parity.host(theta), parity.host(mom)
    orc = oracle.outer_step(theta0, mom0, parity.host(theta_L), stride, tensors, weights, present, LR, BETA,
                            bases=[parity.host(b) for b in bases], rule="rda")
    view = workloads.StepInputs(theta, mom, theta_L, tensors, weights, present, list(range(len(tensors))), stride)
    parity.compare(gpu, orc, view, pinned=False, state=False)
    check_merge_on_gpu_codes(gpu, view, theta0, mom0)


def test_rda_with_theta_g_as_every_base_equals_no_bases():
    inp = make_inputs(41, 5, SIZES, [1.0, 0.0, 2.0, 0.5, 1.5])
    k = inp.theta_L.shape[0]
    a = gpu_rda(inp)
    codes, cb, rng, norms, ws = rda_buffers(k, inp.theta_L.shape[1], len(inp.tensors), inp.tensors)
    th, mo = inp.theta_g.clone(), inp.momentum.clone()
    dlc.dlc_rda_outer_step(th, mo, inp.theta_L, inp.tensors, inp.weights, codes, cb, rng, norms, ws, LR, BETA,
                           bases=[inp.theta_g] * k)
    torch.cuda.synchronize()
    assert torch.equal(th, a["theta"]) and torch.equal(mo, a["momentum"])
    for i in range(k):
        if inp.weights[i] > 0:
            assert torch.equal(cb[i], a["codebook"][i]) and torch.equal(rng[i], a["range"][i])
            assert torch.equal(norms[i], a["sq_norms"][i])


@pytest.mark.slow
def test_rda_full_1b_set_sampled_tensors():
    cfg = workloads.config("c3")
    inp = workloads.fragment_inputs(cfg, list(range(len(cfg.tensors))), DEV)
    k = inp.theta_L.shape[0]
    theta0, mom0 = inp.theta_g.clone(), inp.momentum.clone()
    gpu = gpu_rda(inp)
    sizes = sorted((n, t) for t, (_, _, n) in enumerate(inp.tensors))
    # the smallest tensor, the median one and the largest below 20M elements
    picks = sorted({sizes[0][1], sizes[len(sizes) // 2][1], max((n, t) for n, t in sizes if n <= 20_000_000)[1]})
    w_hat = oracle.normalize_weights(inp.weights)
    present = [i for i, w in enumerate(inp.weights) if w > 0]
    for t in picks:
        off, loff, n = inp.tensors[t]
        cs = [parity.host(gpu["codes"][i, loff:loff + n]) for i in present]
        cbs = [parity.host(gpu["codebook"][i, t]) for i in present]
        for i, c, b in zip(present, cs, cbs):
            x = oracle.dequantize(c, b).astype(np.float64)
            assert abs(float(gpu["sq_norms"][i, t]) - float(np.sum(x * x))) <= 1e-12 * float(np.sum(x * x))
        g = oracle.rda_merge(cs, cbs, [w_hat[i] for i in present])
        th_o, mo_o = oracle.nesterov(parity.host(theta0[off:off + n]), parity.host(mom0[off:off + n]), g, cfg.lr,
                                     cfg.beta)
        assert parity.ulp_distance(parity.host(gpu["theta"][off:off + n]), th_o).max() <= 1
        assert parity.ulp_distance(parity.host(gpu["momentum"][off:off + n]), mo_o).max() <= 1
        print(f"[rda c3] tensor {t} ({n} params, K = {k}) ok", flush=True)


@pytest.mark.parametrize("name", ["mean_dominated_k3", "above_hi_mean_dominated_k2", "tiny_values_k3",
                                  "huge_values_k2"])
def test_rda_norms_from_exact_bucket_counts(name):
    """Pseudo-gradients whose mean dwarfs their spread, some with elements above hi,
    and values near the bottom and the top of the fp32 range (squares far outside
    it): the squared norms come from the bucket counts, so they equal sum_c n_c cb_c^2
    with the oracle's counts n_c (codes identical end to end) and the GPU's entries;
    then the oracle's RDA merge on the GPU's codes gives theta and momentum."""
    inp = case_inputs(name)
    gpu = gpu_rda(inp)
    theta0, mom0 = parity.host(inp.theta_g), parity.host(inp.momentum)
    orc = oracle.outer_step(theta0, mom0, parity.host(inp.theta_L), inp.theta_L.shape[1], inp.tensors, inp.weights,
                            inp.present, LR, BETA, rule="rda")
    rep = parity.compare(gpu, orc, inp, pinned=False, state=False)
    assert rep["flips"] == 0
    cb, norms = parity.host(gpu["codebook"]), parity.host(gpu["sq_norms"])
    for (i, t), q in orc["quant"].items():
        want = float(np.sum(q["bucket_count"] * cb[i, t].astype(np.float64) ** 2))
        assert abs(norms[i, t] - want) <= 1e-12 * want, (i, t, norms[i, t], want)
    check_merge_on_gpu_codes(gpu, inp, theta0, mom0)
