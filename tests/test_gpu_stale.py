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
