"""GPU parity at the largest tensor the C ABI takes (numel = 2^32 - 1, offsets
past 2^32 elements), one learner.

The oracle cannot run over 4.3e9 elements in a test's time, so the check uses
what holds at any size:
  * statistics: the fp64 mean and population deviation of Delta, accumulated
    chunk by chunk on the host about a shift, give the range the oracle's
    clip_range makes from them (within one fp32 ulp of the GPU's);
  * codes: bit-exact against oracle.encode with the GPU's (lo, wd) at sampled
    positions (random ones, both ends of the tensor, the ragged tail);
  * codebook: every used entry lies in its bucket [lo + c wd, lo + (c + 1) wd]
    (up to fp32 rounding), every empty one is its midpoint, and the bucket
    counts (np.bincount of the codes) sum to numel;
  * theta and momentum at the sampled positions: bit-exact against oracle.merge
    and oracle.nesterov on the GPU's codes and codebook;
  * two small tensors around the large one (one past 2^32 elements) against the
    full oracle with the parity bar of tests/parity.py.
"""
import numpy as np
import pytest
import torch

import diloco_outer_step_amd as dlc
import oracle
import workloads
from tests import parity

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

DEV = "cuda"
LR, BETA = 0.7, 0.9
BIG = (1 << 32) - 1
CHUNK = 1 << 28


def test_largest_tensor_one_learner():
    sizes = [5000, BIG, 777]
    tensors, pos = [], 0
    for n in sizes:
        tensors.append((pos, pos, n))
        pos += (n + 63) // 64 * 64
    stride = pos
    assert tensors[2][0] > (1 << 32)
    print(f"[max size] numel {BIG}, stride {stride}", flush=True)
    g = torch.Generator(device=DEV)
    g.manual_seed(77)
    theta = torch.empty(stride, dtype=torch.float32, device=DEV)
    theta_L = torch.empty((1, stride), dtype=torch.float32, device=DEV)
    for a in range(0, stride, CHUNK):  # bounded temporaries
        b = min(stride, a + CHUNK)
        theta[a:b].normal_(0.0, 0.02, generator=g)
        theta_L[0, a:b] = theta[a:b] - torch.randn(b - a, generator=g, device=DEV) * 1e-3
    mom = torch.zeros(stride, dtype=torch.float32, device=DEV)
    theta0 = theta.clone()
    codes, cb, rng = dlc.outputs_for(1, stride, len(tensors), DEV)
    ws = dlc.alloc_workspace(1, tensors, DEV)
    dlc.dlc_quantize(theta, theta_L, tensors, codes, cb, rng, ws)
    dlc.dlc_merge_outer_step(theta, mom, codes, cb, [1.0], tensors, LR, BETA)
    torch.cuda.synchronize()
    print("[max size] GPU step done", flush=True)

    off, loff, n = tensors[1]
    lo, hi, wd, mean32 = (np.float32(v) for v in parity.host(rng[0, 1]))
    # statistics, chunk by chunk about a shift (fp64)
    shift = None
    s1 = s2 = 0.0
    counts = np.zeros(256, np.int64)
    for a in range(0, n, CHUNK):
        b = min(n, a + CHUNK)
        x = np.subtract(parity.host(theta0[off + a:off + b]), parity.host(theta_L[0, loff + a:loff + b]),
                        dtype=np.float32).astype(np.float64)
        if shift is None:
            shift = float(x[0])
        d = x - shift
        s1 += float(np.sum(d))
        s2 += float(np.sum(d * d))
        counts += np.bincount(parity.host(codes[0, loff + a:loff + b]), minlength=256)
    mu = shift + s1 / n
    sigma = float(np.sqrt(max(s2 / n - (s1 / n) ** 2, 0.0)))
    want = oracle.clip_range(mu, sigma)
    for got, ref in zip((lo, hi, wd), want[:3]):
        assert parity.ulp_distance(np.array([got]), np.array([ref]))[0] <= 1, (got, ref)
    assert counts.sum() == n
    print(f"[max size] range ok: mu {mu:.3e} sigma {sigma:.3e}", flush=True)
    # codebook: used entries inside their buckets, empty ones at the midpoint
    cbh = parity.host(cb[0, 1]).astype(np.float64)
    c = np.arange(256)
    left = np.float64(lo) + c * np.float64(wd)
    right = left + np.float64(wd)
    right[255] = max(right[255], np.float64(hi))  # the last bucket also holds the values clipped to hi
    used = counts > 0
    # fp32 bucket assignment can place a value up to ~2^-16 wd outside its exact
    # interval, and the entry itself is rounded to fp32
    slack = np.abs(np.spacing(cbh.astype(np.float32))).astype(np.float64) + np.float64(wd) * 2.0 ** -14
    assert np.all(cbh[used] >= left[used] - slack[used])
    assert np.all(cbh[used] <= right[used] + slack[used])
    mid = oracle.codebook(np.zeros(256), np.zeros(256, np.int64), lo, wd)
    np.testing.assert_array_equal(parity.host(cb[0, 1])[~used], mid[~used])
    # sampled positions: codes, theta, momentum
    rs = np.random.default_rng(5)
    idx = np.unique(np.concatenate([rs.integers(0, n, 1 << 20), np.arange(4096), np.arange(n - 70000, n)]))
    it = torch.from_numpy(idx).to(DEV)
    x = np.subtract(parity.host(theta0[off + it]), parity.host(theta_L[0, loff + it]), dtype=np.float32)
    code_s = parity.host(codes[0, loff + it])
    np.testing.assert_array_equal(code_s, oracle.encode(x, lo, wd))
    gs = oracle.merge([code_s], [parity.host(cb[0, 1])], [1.0])
    th_o, mo_o = oracle.nesterov(parity.host(theta0[off + it]), np.zeros(len(idx), np.float32), gs, LR, BETA)
    np.testing.assert_array_equal(parity.host(theta[off + it]), th_o)
    np.testing.assert_array_equal(parity.host(mom[off + it]), mo_o)
    print(f"[max size] {len(idx)} sampled elements bit-exact", flush=True)
    # the two small tensors, the second one past 2^32 elements
    for t in (0, 2):
        o, lo_, m = tensors[t]
        width = (m + 63) // 64 * 64
        pad = torch.zeros((1, width), dtype=torch.float32, device=DEV)
        pad[:, :m] = theta_L[:, lo_:lo_ + m]
        view = workloads.StepInputs(theta0[o:o + m].clone(), torch.zeros(m, device=DEV), pad, [(0, 0, m)], [1.0],
                                    [1], [0], width)
        gpu = dict(codes=torch.zeros((1, width), dtype=torch.uint8, device=DEV), codebook=cb[:, t:t + 1],
                   range=rng[:, t:t + 1], theta=theta[o:o + m], momentum=mom[o:o + m])
        gpu["codes"][:, :m] = codes[:, lo_:lo_ + m]
        parity.compare(gpu, parity.oracle_step(view, LR, BETA), view, pinned=False)
