"""GPU parity on seeded random parameter sets.

Tensor sizes are drawn around the edges of the block partition (the 64-element
alignment, tiles of 4096 elements, encode groups of 4 tiles, the 28-tile cap of an
encode block) or uniformly; 1 to 17 learners (across the 14-learner statistics
launch and the 16-learner encode launch), some absent, with equal or Dirichlet
weights; Gaussian, Laplace or Student-t pseudo-gradients of scale 1e-4 to 1e-2;
some constant tensors (the zero-variance path).  Every set runs the whole step
through the C ABI and is compared with the oracle at the parity bar of
tests/parity.py: end to end, and given the oracle's ranges (codes bit-exact).
Half of the sets also run Radial-Directional Averaging (the bar of
tests/test_gpu_rda.py); a third of them whole fragment cycles on one to four
lanes, with and without sending the update back, merged by the weighted mean and
(every other set) by Radial-Directional Averaging, against fragment-by-fragment
calls (bit-identical, as in tests/test_gpu_cycle.py); a third of them learners
on one to three older bases (dlc_quantize_bases, the parity bar above); and the
sets whose learners are all present the requantizing ring (the per-chunk checks
of tests/test_gpu_ring.py, with at most a tenth of the chunks diverging, each from
an adjacent-bucket flip).
"""
import numpy as np
import pytest
import torch

import diloco_outer_step_amd as dlc
import oracle
import workloads
from tests import parity
from tests.test_gpu_cycle import assert_same, run_cycle, run_cycle_rda, run_sequential, run_sequential_rda
from tests.test_gpu_rda import check_merge_on_gpu_codes, gpu_rda
from tests.test_gpu_ring import check_against_oracle, check_divergence_origins, gpu_ring

pytestmark = pytest.mark.gpu

DEV = "cuda"
EDGES = [1, 2, 63, 64, 65, 1000, 4095, 4096, 4097, 8192, 12289, 16383, 16384, 16385,
         28 * 4096 - 1, 28 * 4096, 28 * 4096 + 1, 29 * 4096 + 5]
SEEDS = list(range(24))


def random_config(seed):
    """(config, sizes, kinds, delta, scale, weights) of random set `seed`."""
    rng = np.random.default_rng(1000 + seed)
    k = int(rng.choice([1, 2, 3, 4, 7, 8, 13, 15, 16, 17]))
    n_t = int(rng.integers(1, 13))
    sizes = [int(rng.choice(EDGES)) if rng.random() < 0.75 else int(rng.integers(1, 150_000)) for _ in range(n_t)]
    kinds = [str(rng.choice(["matrix"] * 6 + ["vector", "const"])) for _ in range(n_t)]
    delta = str(rng.choice(["normal", "laplace", "student_t"]))
    scale = float(10.0 ** rng.uniform(-4.0, -2.0))
    weights = str(rng.choice(["equal", "dirichlet"]))
    absent_p = float(rng.choice([0.0, 0.25]))
    cfg = workloads.custom(f"random_{seed}", sizes, k, delta=delta, delta_scale=scale, weights=weights,
                           absent_p=absent_p, kinds=kinds)
    return cfg, sizes, kinds, delta, scale, weights


def random_set(seed, device=DEV):
    """(inputs, description) of random set `seed`."""
    cfg, sizes, kinds, delta, scale, weights = random_config(seed)
    inp = workloads.fragment_inputs(cfg, list(range(len(sizes))), device, step=seed + 1, fragment=seed)
    desc = dict(k=cfg.n_learners, sizes=sizes, kinds=kinds, delta=delta, scale=round(scale, 6), weights=weights,
                present=inp.present)
    return inp, desc


@pytest.mark.parametrize("seed", SEEDS)
def test_random_set_against_the_oracle(seed):
    inp, desc = random_set(seed)
    print(f"[random set {seed}] {desc}", flush=True)
    orc = parity.oracle_step(inp)
    rep = parity.compare(parity.gpu_step(inp), orc, inp, pinned=False)
    r, _ = parity.oracle_ranges_tensor(orc, inp)
    rep_pinned = parity.compare(parity.gpu_step(inp, given_range=r.to(DEV)), orc, inp, pinned=True)
    print(f"[random set {seed}] end to end {rep}; given the oracle's ranges {rep_pinned}", flush=True)


@pytest.mark.parametrize("seed", SEEDS[::2])
def test_random_set_rda(seed):
    inp, desc = random_set(seed)
    print(f"[random set {seed}, RDA] {desc}", flush=True)
    gpu = gpu_rda(inp)
    theta0, mom0 = parity.host(inp.theta_g), parity.host(inp.momentum)
    check_merge_on_gpu_codes(gpu, inp, theta0, mom0)
    orc = oracle.outer_step(theta0, mom0, parity.host(inp.theta_L), inp.theta_L.shape[1], inp.tensors, inp.weights,
                            inp.present, 0.7, 0.9, rule="rda")
    rep = parity.compare(gpu, orc, inp, pinned=False, state=False)
    print(f"[random set {seed}, RDA] quantization {rep}", flush=True)


@pytest.mark.parametrize("seed", SEEDS[::3])
def test_random_set_cycle(seed):
    inp, desc = random_set(seed)
    rng = np.random.default_rng(2000 + seed)
    sizes = [n for _, _, n in inp.tensors]
    n_fragments = int(rng.integers(2, 6))
    frag, _ = dlc.dlc_fragment_plan(sizes, n_fragments)
    grouped, first, _ = dlc.group_by_fragment(inp.tensors, frag, n_fragments)
    k = len(inp.present)
    weights = []
    for _ in range(n_fragments):
        w = [float(x) if p else 0.0 for x, p in zip(rng.uniform(0.5, 2.0, k), inp.present)]
        for i in range(k):
            if rng.random() < 0.3:
                w[i] = 0.0
        if not any(x > 0 for x in w):
            w[inp.present.index(1)] = 1.0
        weights.append(w)
    n_lanes = int(rng.integers(1, 5))
    broadcast = bool(rng.integers(0, 2))
    print(f"[random set {seed}, cycle] {desc}, {n_fragments} fragments, {n_lanes} lanes, send back {broadcast}",
          flush=True)
    mom = torch.randn(inp.momentum.shape, generator=torch.Generator(device=DEV).manual_seed(seed), device=DEV) * 1e-3
    args = (inp.theta_g, mom, inp.theta_L, grouped, first, weights)
    lanes = [None] + [torch.cuda.Stream() for _ in range(n_lanes - 1)]
    a = run_cycle(*args, broadcast=broadcast, two_streams=False, lanes=lanes)
    b = run_sequential(*args, broadcast=broadcast)
    assert_same(a, b, weights, grouped, first)
    if seed % 2 == 0:  # the same cycle merged by Radial-Directional Averaging
        a = run_cycle_rda(*args, broadcast=broadcast, lanes=lanes)
        b = run_sequential_rda(*args, broadcast=broadcast)
        assert_same(a, b, weights, grouped, first)
        for f in range(n_fragments):
            for i, w in enumerate(weights[f]):
                if w > 0:
                    assert torch.equal(a["sq_norms"][i, first[f]:first[f + 1]], b["sq_norms"][i, first[f]:first[f + 1]])


@pytest.mark.parametrize("seed", SEEDS[1::3])
def test_random_set_stale_bases(seed):
    inp, desc = random_set(seed)
    rng = np.random.default_rng(3000 + seed)
    k = len(inp.present)
    gen = torch.Generator(device=DEV).manual_seed(3000 + seed)
    old1 = inp.theta_g - torch.randn(inp.theta_g.shape, generator=gen, device=DEV) * 2e-3
    old2 = old1 - torch.randn(inp.theta_g.shape, generator=gen, device=DEV) * 2e-3
    versions = [int(v) for v in rng.integers(0, 3, k)]
    base_of = [inp.theta_g, old1, old2]
    bases = [base_of[v] for v in versions]
    # learner i started from its base: the same pseudo-gradient, against that base
    theta_L = torch.stack([bases[i] - (inp.theta_g - inp.theta_L[i]) for i in range(k)]).contiguous()
    print(f"[random set {seed}, stale] {desc}, bases {versions}", flush=True)
    stride = theta_L.shape[1]
    codes, cb, rg = dlc.outputs_for(k, stride, len(inp.tensors), DEV)
    ws = dlc.alloc_workspace(k, inp.tensors, DEV)
    th, mo = inp.theta_g.clone(), inp.momentum.clone()
    dlc.dlc_quantize_bases(bases, theta_L, inp.tensors, codes, cb, rg, ws, present=inp.present)
    dlc.dlc_merge_outer_step(th, mo, codes, cb, inp.weights, inp.tensors)
    torch.cuda.synchronize()
    orc = oracle.outer_step(parity.host(inp.theta_g), parity.host(inp.momentum), parity.host(theta_L), stride,
                            inp.tensors, inp.weights, inp.present, bases=[parity.host(b) for b in bases])
    view = workloads.StepInputs(inp.theta_g, inp.momentum, theta_L, inp.tensors, inp.weights, inp.present,
                                inp.tensor_ids, stride)
    rep = parity.compare(dict(codes=codes, codebook=cb, range=rg, theta=th, momentum=mo), orc, view, pinned=False)
    print(f"[random set {seed}, stale] {rep}", flush=True)


# the ring has no absent ranks: the sets whose learners are all present
RING_SEEDS = [s for s in SEEDS if all(workloads.presence(random_config(s)[0], s))][:8]


@pytest.mark.parametrize("seed", RING_SEEDS)
def test_random_set_ring(seed):
    inp, desc = random_set(seed)
    k = len(inp.present)
    print(f"[random set {seed}, ring] {desc}", flush=True)
    mom = torch.randn(inp.momentum.shape, generator=torch.Generator(device=DEV).manual_seed(seed), device=DEV) * 1e-3
    th, _, codes, _ = gpu_ring(inp.theta_g, mom, inp.theta_L, inp.tensors, messages=True)
    theta0, tl = parity.host(inp.theta_g), parity.host(inp.theta_L)
    orc = oracle.ring_outer_step(theta0, parity.host(mom), tl, inp.theta_L.shape[1], inp.tensors, 0.7, 0.9)
    diverged, chunks = check_against_oracle(parity.host(th), orc, theta0, tl, inp.tensors, k)
    origins = check_divergence_origins(codes, orc, inp.tensors, k, check_against_oracle.diverged)
    print(f"[random set {seed}, ring] {diverged} of {chunks} chunks diverged, first differing hops {origins}",
          flush=True)
    assert diverged <= chunks // 10
