"""Helpers shared by the parity tests: run one outer step through the C ABI and
through the CPU oracle on the same inputs, and compare the two.

Tolerances (stated once, used everywhere):
  * codes: bit-exact when the GPU is handed the oracle's (lo, hi, wd, mean);
    end to end, at most 1e-6 of the elements may differ and only to an adjacent
    bucket;
  * codebooks: within one fp32 ulp plus wd * 2^-25 of the oracle's fp64 bucket
    means (the GPU accumulates bucket positions in 2^-26 wd fixed point);
  * theta and momentum: |gpu - oracle| <= 1e-9 + 1e-5 |oracle| on every element
    whose K codes all equal the oracle's; where a code flipped, the change of
    theta is bounded by the codebook step it causes.
"""
from __future__ import annotations

import numpy as np
import torch

import diloco_outer_step_amd as dlc
import oracle

RTOL = 1e-5
ATOL = 1e-9
MAX_FLIP_FRACTION = 1e-6


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()


def gpu_step(inp, lr=0.7, beta=0.9, given_range=None, merge=True, stream=None):
    """One quantize + merge call through the C ABI on copies of inp's state."""
    k, stride = inp.theta_L.shape
    t = len(inp.tensors)
    dev = inp.theta_L.device
    codes, cb, rng = dlc.outputs_for(k, stride, t, dev)
    ws = dlc.alloc_workspace(k, inp.tensors, dev)
    theta = inp.theta_g.clone()
    mom = inp.momentum.clone()
    if given_range is not None:
        rng.copy_(given_range)
    dlc.dlc_quantize(inp.theta_g, inp.theta_L, inp.tensors, codes, cb, rng, ws,
                     present=inp.present, range_given=given_range is not None, stream=stream)
    if merge:
        dlc.dlc_merge_outer_step(theta, mom, codes, cb, inp.weights, inp.tensors, lr, beta, stream=stream)
    torch.cuda.synchronize()
    return dict(codes=codes, codebook=cb, range=rng, theta=theta, momentum=mom)


def oracle_step(inp, lr=0.7, beta=0.9, given_ranges=None):
    return oracle.outer_step(host(inp.theta_g), host(inp.momentum), host(inp.theta_L),
                             inp.theta_L.shape[1], inp.tensors, inp.weights, inp.present, lr, beta,
                             given_ranges)


def oracle_ranges_tensor(orc, inp):
    """The oracle's (lo, hi, wd, mean) per (learner, tensor) as a [K, T, 4] tensor,
    plus the dict form the oracle takes back."""
    k = inp.theta_L.shape[0]
    t = len(inp.tensors)
    r = torch.zeros((k, t, 4), dtype=torch.float32)
    given = {}
    for (i, ti), q in orc["quant"].items():
        vals = (q["lo"], q["hi"], q["wd"], q["mean32"])
        r[i, ti] = torch.tensor([float(v) for v in vals], dtype=torch.float32)
        given[(i, ti)] = vals
    return r, given


def codebook_bound(cb_oracle, wd):
    """Largest allowed |codebook_gpu - codebook_oracle| per entry.

    The GPU sums each element's position inside its bucket as an integer in units
    of wd * 2^-26 (rounded to nearest), so a bucket mean is off by at most
    wd * 2^-27 before both sides round to fp32: one fp32 ulp of the entry plus
    wd * 2^-25 covers it with margin."""
    cb = np.asarray(cb_oracle, np.float32)
    return np.abs(np.spacing(cb)).astype(np.float64) + float(wd) * 2.0 ** -25


def ulp_distance(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Distance in fp32 units in the last place (ordered-integer metric)."""
    def key(x):
        i = np.asarray(x, np.float32).view(np.int32).astype(np.int64)
        return np.where(i < 0, -(i & 0x7FFFFFFF), i)
    return np.abs(key(a) - key(b))


def compare(gpu, orc, inp, pinned: bool, report: dict | None = None, state: bool = True):
    """Assert parity; returns a report dict (flip counts, exact fractions, ulp stats).
    state=False checks the quantization outputs only (codes, codebooks, ranges)."""
    rep = dict(elements=0, flips=0, range_ulp_max=0, cb_ulp_max=0, theta_exact=0, mom_exact=0,
               pairs=0, range_exact_pairs=0)
    codes_g = host(gpu["codes"])
    cb_g = host(gpu["codebook"])
    rng_g = host(gpu["range"])
    theta_g, mom_g = host(gpu["theta"]), host(gpu["momentum"])
    for ti, (off, loff, n) in enumerate(inp.tensors):
        all_match = np.ones(n, bool)
        flip_bound = np.zeros(n, np.float64)
        w_hat = oracle.normalize_weights(inp.weights)
        for i in range(inp.theta_L.shape[0]):
            if not inp.present[i]:
                continue
            q = orc["quant"][(i, ti)]
            ro = np.array([q["lo"], q["hi"], q["wd"], q["mean32"]], np.float32)
            d = ulp_distance(rng_g[i, ti], ro)
            rep["pairs"] += 1
            rep["range_exact_pairs"] += int(d.max() == 0)
            rep["range_ulp_max"] = max(rep["range_ulp_max"], int(d[:3].max()))
            if pinned:
                assert d.max() == 0, f"range changed in pinned mode (learner {i}, tensor {ti})"
            cg = codes_g[i, loff:loff + n]
            co = q["codes"]
            mism = cg != co
            nm = int(mism.sum())
            rep["elements"] += n
            rep["flips"] += nm
            if pinned:
                assert nm == 0, f"{nm} code mismatches given the oracle's range (learner {i}, tensor {ti})"
            if nm:
                diff = np.abs(cg[mism].astype(np.int64) - co[mism].astype(np.int64))
                assert diff.max() <= 1, f"non-adjacent code flip (learner {i}, tensor {ti})"
                all_match &= ~mism
                cbg, cbo = cb_g[i, ti], q["codebook"]
                step = np.abs(cbg[cg].astype(np.float64) - cbo[co].astype(np.float64))
                flip_bound += w_hat[i] * step
            if d[:3].max() == 0:
                used = q["bucket_count"] > 0
                u = ulp_distance(cb_g[i, ti], q["codebook"])
                rep["cb_ulp_max"] = max(rep["cb_ulp_max"], int(u[used].max()) if used.any() else 0)
                err = np.abs(cb_g[i, ti].astype(np.float64) - q["codebook"].astype(np.float64))
                bound = codebook_bound(q["codebook"], q["wd"])
                assert np.all(err[used] <= bound[used]), \
                    f"codebook outside its bound (learner {i}, tensor {ti}): max err {err[used].max():.3e}"
        if not state:
            continue
        th_o = orc["theta"][off:off + n].astype(np.float64)
        mo_o = orc["momentum"][off:off + n].astype(np.float64)
        th_gv = theta_g[off:off + n].astype(np.float64)
        mo_gv = mom_g[off:off + n].astype(np.float64)
        ok_th = np.abs(th_gv - th_o) <= ATOL + RTOL * np.abs(th_o)
        ok_mo = np.abs(mo_gv - mo_o) <= ATOL + RTOL * np.abs(mo_o)
        bad = all_match & ~(ok_th & ok_mo)
        assert not bad.any(), (f"theta/momentum outside tolerance at {int(bad.sum())} elements of tensor {ti}; "
                               f"max |dtheta| {np.max(np.abs(th_gv - th_o)[bad]):.3e}")
        if (~all_match).any():
            lr_beta = 0.7 * (1 + 0.9)
            fl = ~all_match
            assert np.all(np.abs(th_gv - th_o)[fl] <= lr_beta * flip_bound[fl] * 1.01 + ATOL + RTOL * np.abs(th_o[fl]))
        rep["theta_exact"] += int(np.sum(th_gv == th_o))
        rep["mom_exact"] += int(np.sum(mo_gv == mo_o))
    if not pinned and rep["elements"]:
        assert rep["flips"] <= MAX_FLIP_FRACTION * rep["elements"] + 0.5, \
            f"{rep['flips']} code flips in {rep['elements']} elements"
    if report is not None:
        report.update(rep)
    return rep
