"""GPU tests of the ring with requantization at every hop (dlc_ring_outer_step)
against the CPU oracle's ring_outer_step.

* one rank: bit-identical to the star path (dlc_quantize + a one-learner merge);
* constant chunks (every message lossless): bit-identical to the oracle,
  including the fp32 ring-order sums and the division by K;
* Gaussian pseudo-gradients (K up to 16): the GPU's codebooks may differ from
  the oracle's by an ulp, which can move a later hop's code to the neighbouring
  bucket; that chunk's later sums, ranges and codes then differ too (the ring
  requantizes what it received).  The bar: per chunk, either 99.9% of theta
  within 1e-9 + 1e-5 |theta| or the chunk counts as diverged; at most a tenth of
  the chunks diverge; every element within the bucket widths the messages can
  shift it by; and the GPU's g within 5% (RMS) of the exact mean's scale from
  the oracle's g.
"""
import numpy as np
import pytest
import torch

import diloco_outer_step_amd as dlc
import oracle

pytestmark = pytest.mark.gpu

DEV = "cuda"
LR, BETA = 0.7, 0.9


def packed(sizes):
    offs, pos = [], 0
    for n in sizes:
        offs.append(pos)
        pos += (n + 63) // 64 * 64
    return [(o, o, n) for o, n in zip(offs, sizes)], pos


def gpu_ring(theta, mom, theta_L, tensors):
    th, mo = theta.clone(), mom.clone()
    accum, codes, cb, rng = dlc.ring_buffers(theta_L, len(tensors))
    ws = torch.empty(max(256, dlc.dlc_ring_workspace_bytes(theta_L.shape[0], tensors)), dtype=torch.uint8,
                     device=DEV)
    dlc.dlc_ring_outer_step(th, mo, theta_L, tensors, accum, codes, cb, rng, ws, LR, BETA)
    torch.cuda.synchronize()
    return th, mo


def host(t):
    return t.cpu().numpy()


def test_one_rank_equals_the_star_path():
    tensors, stride = packed([5000, 4096 * 3 + 1, 64, 100003])
    g = torch.Generator(device=DEV)
    g.manual_seed(3)
    theta = torch.randn(stride, generator=g, device=DEV) * 0.02
    mom = torch.randn(stride, generator=g, device=DEV) * 1e-3
    theta_L = (theta - torch.randn(stride, generator=g, device=DEV) * 1e-3).reshape(1, stride).contiguous()
    th, mo = gpu_ring(theta, mom, theta_L, tensors)
    codes, cb, rng = dlc.outputs_for(1, stride, len(tensors), DEV)
    ws = dlc.alloc_workspace(1, tensors, DEV)
    th2, mo2 = theta.clone(), mom.clone()
    dlc.dlc_quantize(theta, theta_L, tensors, codes, cb, rng, ws)
    dlc.dlc_merge_outer_step(th2, mo2, codes, cb, [1.0], tensors, LR, BETA)
    torch.cuda.synchronize()
    assert torch.equal(th, th2) and torch.equal(mo, mo2)


@pytest.mark.parametrize("k", [2, 3, 5, 8, 64])
def test_constant_chunks_bit_exact(k):
    sizes = [64 * 7 + 5, 4096 * 2, 100, 64 * 40]
    tensors, stride = packed(sizes)
    rng = np.random.default_rng(k)
    theta = np.ones(stride, np.float32)
    tl = np.ones((k, stride), np.float32)
    for _, lo, n in tensors:
        for c, (a, b) in enumerate(oracle.ring_chunks(n, k)):
            for r in range(k):
                tl[r, lo + a:lo + b] = np.float32(1.0) - np.float32(rng.uniform(-1e-3, 1e-3))
    mom = (rng.standard_normal(stride) * 1e-3).astype(np.float32)
    th, mo = gpu_ring(torch.from_numpy(theta).to(DEV), torch.from_numpy(mom).to(DEV),
                      torch.from_numpy(tl).to(DEV), tensors)
    orc = oracle.ring_outer_step(theta, mom, tl, stride, tensors, LR, BETA)
    for o, _, n in tensors:
        np.testing.assert_array_equal(host(th)[o:o + n], orc["theta"][o:o + n])
        np.testing.assert_array_equal(host(mo)[o:o + n], orc["momentum"][o:o + n])


@pytest.mark.parametrize("k", [2, 4, 8, 16])
def test_gaussian_against_oracle(k):
    sizes = [64 * 300 + 9, 4096 * 8, 50000]
    tensors, stride = packed(sizes)
    g = torch.Generator(device=DEV)
    g.manual_seed(10 + k)
    theta = torch.randn(stride, generator=g, device=DEV) * 0.02
    mom = torch.randn(stride, generator=g, device=DEV) * 1e-3
    theta_L = torch.stack([theta - torch.randn(stride, generator=g, device=DEV) * 1e-3 for _ in range(k)])
    th, mo = gpu_ring(theta, mom, theta_L, tensors)
    orc = oracle.ring_outer_step(host(theta), host(mom), host(theta_L), stride, tensors, LR, BETA)
    th_g, th_o = host(th).astype(np.float64), orc["theta"].astype(np.float64)
    diverged = chunks = 0
    for t, (o, lo, n) in enumerate(tensors):
        wd = max(float(q["wd"]) for (tt, _, _, _, q) in orc["messages"] if tt == t)
        for a, b in oracle.ring_chunks(n, k):
            if b <= a:
                continue
            chunks += 1
            d = np.abs(th_g[o + a:o + b] - th_o[o + a:o + b])
            ok = d <= 1e-9 + 1e-5 * np.abs(th_o[o + a:o + b])
            # A code that lands on the other side of a bucket edge (the two sides' codebooks
            # may differ by an ulp) changes that chunk's later sums, ranges and codes: the
            # chunk then diverges, but only by the bucket widths the messages can shift it.
            if ok.mean() < 0.999:
                diverged += 1
            assert d.max() <= LR * (1 + BETA) * 2.0 * wd, f"tensor {t} chunk [{a}, {b}): max |dtheta| {d.max():.3e}"
        # both rings are equally far from the exact mean of the pseudo-gradients
        exact = np.mean([host(theta)[o:o + n].astype(np.float64)
                         - host(theta_L)[r, lo:lo + n].astype(np.float64) for r in range(k)], 0)
        ref = host(theta)[o:o + n].astype(np.float64)
        g_gpu = (ref - th_g[o:o + n]) / LR  # g + beta v_new, same v for both
        g_orc = (ref - th_o[o:o + n]) / LR
        e_gpu = np.sqrt(np.mean((g_gpu - g_orc) ** 2))
        assert e_gpu <= 0.05 * np.sqrt(np.mean(exact ** 2))
    # divergence is the exception (none at all for K <= 8 on these inputs)
    assert diverged <= max(1, chunks // 10), f"{diverged} of {chunks} chunks diverged"
