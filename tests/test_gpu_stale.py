"""GPU parity for learners that report against older bases (dlc_quantize_bases),
merged with token weights chosen by dlc_merge_weights (Decoupled DiLoCo digest,
"fault tolerance" items 1-3), against the CPU oracle."""
import math

import numpy as np
import pytest
import torch

import diloco_outer_step_amd as dlc
import oracle
import workloads
from tests import parity

pytestmark = pytest.mark.gpu

DEV = "cuda"


def stale_inputs(seed, k=6, sizes=(5000, 4096 * 5 + 3, 64 * 77, 100003, 4096)):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    offs, pos = [], 0
    for n in sizes:
        offs.append(pos)
        pos += (n + 63) // 64 * 64
    tensors = [(o, o, n) for o, n in zip(offs, sizes)]
    theta = torch.randn(pos, generator=g, device=DEV) * 0.02
    # two older versions of the global parameters
    old1 = theta - torch.randn(pos, generator=g, device=DEV) * 2e-3
    old2 = old1 - torch.randn(pos, generator=g, device=DEV) * 2e-3
    version = [0, 1, 0, 2, 1, 0][:k]
    base_of = [theta, old1, old2]
    theta_L = torch.stack([base_of[v] - torch.randn(pos, generator=g, device=DEV) * 1e-3 for v in version])
    mom = torch.randn(pos, generator=g, device=DEV) * 1e-3
    return theta, mom, theta_L.contiguous(), tensors, [base_of[v] for v in version]


def test_stale_bases_against_oracle_with_token_weights():
    theta, mom, theta_L, tensors, bases = stale_inputs(1)
    k, stride = theta_L.shape
    tokens = [4096.0 * (i + 1) for i in range(k)]
    arrival = [0.5, 1.0, 2.5, 0.7, math.inf, 1.9]
    weights, _ = dlc.dlc_merge_weights(tokens, arrival, 3, 1.0)  # quorum at t = 1.0, deadline 2.0
    present = [1 if w > 0 else 0 for w in weights]
    assert present == [1, 1, 0, 1, 0, 1]
    codes, cb, rng = dlc.outputs_for(k, stride, len(tensors), DEV)
    ws = dlc.alloc_workspace(k, tensors, DEV)
    th, mo = theta.clone(), mom.clone()
    dlc.dlc_quantize_bases(bases, theta_L, tensors, codes, cb, rng, ws, present=present)
    dlc.dlc_merge_outer_step(th, mo, codes, cb, weights, tensors)
    torch.cuda.synchronize()
    orc = oracle.outer_step(theta.cpu().numpy(), mom.cpu().numpy(), theta_L.cpu().numpy(), stride, tensors, weights,
                            present, bases=[b.cpu().numpy() for b in bases])
    view = workloads.StepInputs(theta, mom, theta_L, tensors, weights, present, list(range(len(tensors))), stride)
    rep = parity.compare(dict(codes=codes, codebook=cb, range=rng, theta=th, momentum=mo), orc, view, pinned=False)
    assert rep["elements"] > 0


def test_single_base_equals_dlc_quantize():
    theta, mom, theta_L, tensors, _ = stale_inputs(2)
    k, stride = theta_L.shape
    ws = dlc.alloc_workspace(k, tensors, DEV)
    a = dlc.outputs_for(k, stride, len(tensors), DEV)
    b = dlc.outputs_for(k, stride, len(tensors), DEV)
    a[0].zero_()  # the alignment padding between tensors is never written
    b[0].zero_()
    dlc.dlc_quantize(theta, theta_L, tensors, a[0], a[1], a[2], ws)
    dlc.dlc_quantize_bases([theta] * k, theta_L, tensors, b[0], b[1], b[2], ws)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


@pytest.mark.slow
def test_stale_full_1b_set_sampled_tensors():
    """The 1B set at K = 8, odd learners against an older theta, token weights with
    one learner past the merge deadline, every tensor in one call as the bench
    times it; sampled tensors against the oracle one by one (a tensor's results
    depend on that tensor only)."""
    from types import SimpleNamespace
    cfg = workloads.config("c3")
    inp = workloads.fragment_inputs(cfg, list(range(len(cfg.tensors))), DEV)
    k, stride = inp.theta_L.shape
    g = torch.Generator(device=DEV)
    g.manual_seed(5)
    old = inp.theta_g - torch.randn(inp.theta_g.shape, generator=g, device=DEV) * 1e-3
    bases = [inp.theta_g if i % 2 == 0 else old for i in range(k)]
    tokens = [1000.0 * (i + 1) for i in range(k)]
    arrival = [0.1 * i for i in range(k)]
    arrival[3] = 5.0
    weights, _ = dlc.dlc_merge_weights(tokens, arrival, k - 2, 0.5)
    present = [1 if w > 0 else 0 for w in weights]
    assert present == [1, 1, 1, 0, 1, 1, 1, 1]
    codes, cb, rng = dlc.outputs_for(k, stride, len(inp.tensors), DEV)
    ws = dlc.alloc_workspace(k, inp.tensors, DEV)
    th, mo = inp.theta_g.clone(), inp.momentum.clone()
    dlc.dlc_quantize_bases(bases, inp.theta_L, inp.tensors, codes, cb, rng, ws, present=present)
    dlc.dlc_merge_outer_step(th, mo, codes, cb, weights, inp.tensors, cfg.lr, cfg.beta)
    torch.cuda.synchronize()
    sizes = sorted((n, t) for t, (_, _, n) in enumerate(inp.tensors))
    # the smallest tensor, the median one and the largest below 5M elements
    picks = sorted({sizes[0][1], sizes[len(sizes) // 2][1], max((n, t) for n, t in sizes if n <= 5_000_000)[1]})
    for t in picks:
        off, loff, n = inp.tensors[t]
        sn = (n + 63) // 64 * 64
        tl = np.zeros((k, sn), np.float32)
        for i in range(k):
            if present[i]:
                tl[i, :n] = parity.host(inp.theta_L[i, loff:loff + n])
        bs = [parity.host(b[off:off + n]) for b in bases]
        orc = oracle.outer_step(parity.host(inp.theta_g[off:off + n]), parity.host(inp.momentum[off:off + n]), tl,
                                sn, [(0, 0, n)], weights, present, cfg.lr, cfg.beta, bases=bs)
        gc = torch.zeros((k, sn), dtype=torch.uint8)
        gc[:, :n] = codes[:, loff:loff + n].cpu()
        gpu = dict(codes=gc, codebook=cb[:, t:t + 1], range=rng[:, t:t + 1], theta=th[off:off + n],
                   momentum=mo[off:off + n])
        view = SimpleNamespace(theta_L=tl, tensors=[(0, 0, n)], weights=weights, present=present)
        rep = parity.compare(gpu, orc, view, pinned=False)
        print(f"[stale c3] tensor {t} ({n} params): flips {rep['flips']}, theta exact {rep['theta_exact']}/{n}",
              flush=True)
