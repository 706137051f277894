"""GPU parity on seeded random parameter sets.

Tensor sizes are drawn around the edges of the block partition (the 64-element
alignment, tiles of 4096 elements, encode groups of 4 tiles, the 28-tile cap of an
encode block) or uniformly; 1 to 17 learners (across the 14-learner statistics
launch and the 16-learner encode launch), some absent, with equal or Dirichlet
weights; Gaussian, Laplace or Student-t pseudo-gradients of scale 1e-4 to 1e-2;
some constant tensors (the zero-variance path).  Every set runs the whole step
through the C ABI and is compared with the oracle at the parity bar of
tests/parity.py: end to end, and given the oracle's ranges (codes bit-exact).
"""
import numpy as np
import pytest

import workloads
from tests import parity

pytestmark = pytest.mark.gpu

DEV = "cuda"
EDGES = [1, 2, 63, 64, 65, 1000, 4095, 4096, 4097, 8192, 12289, 16383, 16384, 16385,
         28 * 4096 - 1, 28 * 4096, 28 * 4096 + 1, 29 * 4096 + 5]
SEEDS = list(range(24))


def random_set(seed, device=DEV):
    """(inputs, description) of random set `seed`."""
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
    inp = workloads.fragment_inputs(cfg, list(range(n_t)), device, step=seed + 1, fragment=seed)
    desc = dict(k=k, sizes=sizes, kinds=kinds, delta=delta, scale=round(scale, 6), weights=weights,
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
