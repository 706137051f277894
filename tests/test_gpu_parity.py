"""GPU parity: the HIP path through the C ABI against the CPU oracle, element by
element, on the same seeded inputs (tolerances in tests/parity.py)."""
import numpy as np
import pytest
import torch

import diloco_outer_step_amd as dlc
import oracle
import workloads
from tests import edge_inputs, parity

pytestmark = pytest.mark.gpu

DEV = "cuda"

RAGGED = [1, 63, 64, 65, 577, 4095, 4096, 4097, 12289, 100003]


def case_inputs(name):
    if name == "c1":
        cfg = workloads.config("c1")
        return workloads.fragment_inputs(cfg, [0], DEV)
    if name == "ragged_k3":
        cfg = workloads.custom("ragged", RAGGED, 3)
        return workloads.fragment_inputs(cfg, list(range(len(RAGGED))), DEV)
    if name == "c2_median_fragment":
        cfg = workloads.config("c2")
        frag, loads = oracle.fragment_plan([s.numel for s in cfg.tensors], 24)
        order = sorted(range(24), key=lambda p: (loads[p], p))
        p = order[12]
        ids = [t for t, f in enumerate(frag) if f == p]
        return workloads.fragment_inputs(cfg, ids, DEV, fragment=p)
    if name == "many_tensors_k20":
        sizes = [4096] * 70 + [64 * 1000 + 64] * 10 + [5000]
        cfg = workloads.custom("many", sizes, 20, delta="laplace", delta_scale=7e-4)
        return workloads.fragment_inputs(cfg, list(range(len(sizes))), DEV)
    if name == "absent_k16_const":
        sizes = [4096] * 6 + [1 << 16] * 3
        kinds = ["vector", "const", "const", "vector", "const", "vector", "matrix", "matrix", "matrix"]
        cfg = workloads.custom("absent", sizes, 16, delta="laplace", delta_scale=7e-4, absent_p=0.25, kinds=kinds)
        return workloads.fragment_inputs(cfg, list(range(len(sizes))), DEV, fragment=3)
    if name == "sparse_k8":
        # pseudo-gradients that are exactly zero on 90% of the elements (rows no
        # learner touched): codes pile into one bucket
        cfg = workloads.custom("sparse", [1 << 20, 4096 * 7 + 5], 8)
        inp = workloads.fragment_inputs(cfg, [0, 1], DEV)
        gen = torch.Generator(device=DEV)
        gen.manual_seed(1234)
        for i in range(8):
            keep = torch.rand(inp.theta_L.shape[1], generator=gen, device=DEV) < 0.1
            for (o, lo, n) in inp.tensors:
                seg = inp.theta_L[i, lo:lo + n]
                seg.copy_(torch.where(keep[lo:lo + n], seg, inp.theta_g[o:o + n]))
        return inp
    if name == "max_learners_k64":
        # the most learners a call takes: several statistics and encode launches
        # per pass, and the merge's run-time learner loop
        sizes = [1, 65, 4097, 12289, 64 * 500 + 3]
        cfg = workloads.custom("k64", sizes, 64, weights="dirichlet", absent_p=0.2)
        return workloads.fragment_inputs(cfg, list(range(len(sizes))), DEV, fragment=1)
    if name == "mean_dominated_k3":
        # pseudo-gradients whose mean dwarfs their spread (|mu|/sigma ~ 1e7 to 5e7): lo and
        # hi round to fp32 steps comparable to sigma, so the last bucket can span ~20 bucket
        # widths (the histogram then keeps fewer fraction bits for the positions), or lo and
        # hi round to the same value while wd stays normal
        sizes = [64 * 1000 + 7, 4096 * 3, 777]
        tensors, stride = [], 0
        for n in sizes:
            tensors.append((stride, stride, n))
            stride += (n + 63) // 64 * 64
        gen = torch.Generator(device=DEV)
        gen.manual_seed(99)
        theta = torch.full((stride,), 2.0, device=DEV)
        mom = torch.zeros(stride, device=DEV)
        theta_L = torch.empty((3, stride), device=DEV)
        for i, sigma in enumerate([3e-8, 2e-8, 1e-7]):
            theta_L[i] = theta - (1.0 + torch.randn(stride, generator=gen, device=DEV) * sigma)
        return workloads.StepInputs(theta, mom, theta_L, tensors, [1.0, 2.0, 1.0], [1, 1, 1], [0, 1, 2], stride)
    if name == "above_hi_mean_dominated_k2":
        return above_hi_inputs()
    if name == "tiny_values_k3":
        # parameters near the bottom of the fp32 range: learner 0's pseudo-gradients
        # are subnormal (its bucket width underflows: the zero-variance path), learner
        # 1's width lands just above FLT_MIN, learner 2's values are tiny but normal;
        # every subtraction must keep subnormal results (no flush to zero)
        sizes = [5000, 4096 * 2 + 7, 64]
        tensors, stride = [], 0
        for n in sizes:
            tensors.append((stride, stride, n))
            stride += (n + 63) // 64 * 64
        gen = torch.Generator(device=DEV)
        gen.manual_seed(77)
        theta = torch.randn(stride, generator=gen, device=DEV) * 1e-36
        mom = torch.zeros(stride, device=DEV)
        theta_L = torch.empty((3, stride), device=DEV)
        for i, scale in enumerate([2e-39, 4e-37, 3e-35]):
            theta_L[i] = theta - torch.randn(stride, generator=gen, device=DEV) * scale
        return workloads.StepInputs(theta, mom, theta_L, tensors, [1.0, 1.0, 2.0], [1, 1, 1], [0, 1, 2], stride)
    if name == "huge_values_k2":
        # parameters near the top of the fp32 range (clip bounds stay finite): fp64
        # statistics, bucket positions and the merge must not overflow
        sizes = [5000, 4096 * 2 + 7]
        tensors, stride = [], 0
        for n in sizes:
            tensors.append((stride, stride, n))
            stride += (n + 63) // 64 * 64
        gen = torch.Generator(device=DEV)
        gen.manual_seed(78)
        theta = torch.randn(stride, generator=gen, device=DEV) * 1e36
        mom = torch.randn(stride, generator=gen, device=DEV) * 1e33
        theta_L = torch.empty((2, stride), device=DEV)
        for i, scale in enumerate([1e34, 1e30]):
            theta_L[i] = theta - torch.randn(stride, generator=gen, device=DEV) * scale
        return workloads.StepInputs(theta, mom, theta_L, tensors, [3.0, 1.0], [1, 1], [0, 1], stride)
    raise KeyError(name)


def above_hi_inputs():
    """Learner 0: tensors whose (hi - lo) / wd is far from 256 (lo == hi, ~195, ~241,
    ~248, ~271) with elements above hi, which the encode codes from their own
    value but clips to hi; learner 1: ordinary Gaussian tensors with outliers.
    theta_g = 0, so Delta = fl32(0 - theta_i) = -theta_i exactly."""
    xs = [edge_inputs.case_input(name, args) for name, args, _ in edge_inputs.CASES]
    tensors, stride = [], 0
    for x in xs:
        tensors.append((stride, stride, x.size))
        stride += (x.size + 63) // 64 * 64
    tl = np.zeros((2, stride), np.float32)
    for t, (x, (_, lo, n)) in enumerate(zip(xs, tensors)):
        tl[0, lo:lo + n] = -x
        tl[1, lo:lo + n] = -edge_inputs.ordinary(100 + t, n)
    theta = torch.zeros(stride, device=DEV)
    return workloads.StepInputs(theta, torch.zeros(stride, device=DEV), torch.from_numpy(tl).to(DEV), tensors,
                                [1.0, 2.0], [1, 1], list(range(len(xs))), stride)


CASES = ["c1", "ragged_k3", "c2_median_fragment", "many_tensors_k20", "absent_k16_const", "sparse_k8",
         "max_learners_k64", "mean_dominated_k3", "above_hi_mean_dominated_k2", "tiny_values_k3",
         "huge_values_k2"]


@pytest.mark.parametrize("name", CASES)
def test_pinned_range_bit_exact(name):
    """Given the oracle's (lo, hi, wd, mean), codes, codebooks, theta and momentum agree."""
    inp = case_inputs(name)
    orc = parity.oracle_step(inp)
    r, given = parity.oracle_ranges_tensor(orc, inp)
    gpu = parity.gpu_step(inp, given_range=r.to(DEV))
    rep = parity.compare(gpu, orc, inp, pinned=True)
    print(f"[{name} pinned] {rep}")


@pytest.mark.parametrize("name", CASES)
def test_end_to_end(name):
    inp = case_inputs(name)
    orc = parity.oracle_step(inp)
    gpu = parity.gpu_step(inp)
    rep = parity.compare(gpu, orc, inp, pinned=False)
    print(f"[{name} e2e] {rep}")


def test_single_learner_weight_one():
    cfg = workloads.custom("k1", [1 << 20, 333], 1)
    inp = workloads.fragment_inputs(cfg, [0, 1], DEV)
    gpu = parity.gpu_step(inp, lr=1.0, beta=0.0)
    orc = parity.oracle_step(inp, lr=1.0, beta=0.0)
    parity.compare(gpu, orc, inp, pinned=False)
    # g = cb[code] exactly, so theta_new = fl32(theta_g - cb[code])
    codes = parity.host(gpu["codes"])[0]
    cb = parity.host(gpu["codebook"])[0]
    tg = parity.host(inp.theta_g)
    for t, (off, loff, n) in enumerate(inp.tensors):
        want = (tg[off:off + n].astype(np.float64) - cb[t][codes[loff:loff + n]].astype(np.float64)).astype(np.float32)
        assert np.array_equal(parity.host(gpu["theta"])[off:off + n], want)


def test_stages_equal_fused_and_deterministic():
    inp = case_inputs("ragged_k3")
    k, stride = inp.theta_L.shape
    t = len(inp.tensors)
    a = parity.gpu_step(inp, merge=False)
    b = parity.gpu_step(inp, merge=False)
    codes, cb, rng = dlc.outputs_for(k, stride, t, DEV)
    ws = dlc.alloc_workspace(k, inp.tensors, DEV)
    dlc.dlc_quantize_range(inp.theta_g, inp.theta_L, inp.tensors, rng, ws)
    dlc.dlc_quantize_encode(inp.theta_g, inp.theta_L, inp.tensors, rng, codes, cb, ws)
    torch.cuda.synchronize()
    for x in (b, dict(codes=codes, codebook=cb, range=rng)):
        assert torch.equal(a["range"], x["range"])
        for i in range(k):
            for (o, lo, n) in inp.tensors:
                assert torch.equal(a["codes"][i, lo:lo + n], x["codes"][i, lo:lo + n])
        # integer histograms: the codebook does not depend on the order of the atomics
        assert torch.equal(a["codebook"], x["codebook"])


def test_no_quorum_changes_nothing():
    inp = case_inputs("ragged_k3")
    k, stride = inp.theta_L.shape
    codes, cb, rng = dlc.outputs_for(k, stride, len(inp.tensors), DEV)
    theta = inp.theta_g.clone()
    mom = inp.momentum.clone()
    with pytest.raises(dlc.NoQuorumError):
        dlc.dlc_merge_outer_step(theta, mom, codes, cb, [0.0] * k, inp.tensors)
    torch.cuda.synchronize()
    assert torch.equal(theta, inp.theta_g) and torch.equal(mom, inp.momentum)


def test_fragments_equal_whole_set():
    """Merging per fragment (any order) equals one call over every tensor, bit for bit;
    tensors outside a fragment are untouched."""
    cfg = workloads.config("c2")
    ids = list(range(1, 19))  # two layers
    inp = workloads.fragment_inputs(cfg, ids, DEV)
    whole = parity.gpu_step(inp)
    frag, _ = oracle.fragment_plan([n for _, _, n in inp.tensors], 3)
    theta, mom = inp.theta_g.clone(), inp.momentum.clone()
    k, stride = inp.theta_L.shape
    for p in (1, 2, 0):
        sel = [d for d, f in zip(inp.tensors, frag) if f == p]
        codes, cb, rng = dlc.outputs_for(k, stride, len(sel), DEV)
        ws = dlc.alloc_workspace(k, sel, DEV)
        before = theta.clone()
        dlc.dlc_quantize(theta, inp.theta_L, sel, codes, cb, rng, ws)
        dlc.dlc_merge_outer_step(theta, mom, codes, cb, inp.weights, sel)
        torch.cuda.synchronize()
        mask = torch.ones_like(theta, dtype=torch.bool)
        for (o, lo, n) in sel:
            mask[o:o + n] = False
        assert torch.equal(theta[mask], before[mask])
    assert torch.equal(theta, whole["theta"]) and torch.equal(mom, whole["momentum"])
