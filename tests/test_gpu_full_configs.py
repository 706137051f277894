"""GPU parity at the full sizes of every parameter set, in the call shape the
benchmark times (one quantize-range, one quantize-encode and one merge call over
all tensors of the call).  The oracle checks sampled tensors one by one: a
tensor's statistics, codes, codebooks and update depend on that tensor only, so
each sampled tensor is an exact oracle case (tolerances in tests/parity.py).
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


class TensorView:
    """One tensor of a call, copied to host, in the form tests/parity.compare takes."""

    def __init__(self, inp, t, theta_before, mom_before):
        off, loff, n = inp.tensors[t]
        k = inp.theta_L.shape[0]
        stride = (n + 63) // 64 * 64
        self.theta_g = theta_before[off:off + n].clone()
        self.momentum = mom_before[off:off + n].clone()
        self.theta_L = torch.zeros((k, stride), dtype=torch.float32, device=inp.theta_L.device)
        for i in range(k):
            if inp.present[i]:
                self.theta_L[i, :n] = inp.theta_L[i, loff:loff + n]
        self.tensors = [(0, 0, n)]
        self.weights = inp.weights
        self.present = inp.present
        self.src = (t, off, loff, n)


def run_call(inp, theta, mom, lr, beta):
    """The benchmark's three calls on (theta, mom) in place; returns codes, codebook, range."""
    k, stride = inp.theta_L.shape
    codes, cb, rng = dlc.outputs_for(k, stride, len(inp.tensors), DEV)
    ws = dlc.alloc_workspace(k, inp.tensors, DEV)
    dlc.dlc_quantize_range(theta, inp.theta_L, inp.tensors, rng, ws, present=inp.present)
    dlc.dlc_quantize_encode(theta, inp.theta_L, inp.tensors, rng, codes, cb, ws, present=inp.present)
    dlc.dlc_merge_outer_step(theta, mom, codes, cb, inp.weights, inp.tensors, lr, beta)
    torch.cuda.synchronize()
    return codes, cb, rng


def check_sampled(inp, picks, theta_before, mom_before, theta_after, mom_after, codes, cb, rng, cfg, tag):
    reports = []
    for t in picks:
        view = TensorView(inp, t, theta_before, mom_before)
        _, off, loff, n = view.src
        gpu = dict(codes=torch.zeros_like(view.theta_L, dtype=torch.uint8), codebook=cb[:, t:t + 1],
                   range=rng[:, t:t + 1], theta=theta_after[off:off + n], momentum=mom_after[off:off + n])
        gpu["codes"][:, :n] = codes[:, loff:loff + n]
        orc = parity.oracle_step(view, cfg.lr, cfg.beta)
        rep = parity.compare(gpu, orc, view, pinned=False)
        reports.append((t, n, rep))
        print(f"[{tag}] tensor {t} ({n} params): flips {rep['flips']}, range ulp max {rep['range_ulp_max']}, "
              f"codebook ulp max {rep['cb_ulp_max']}, theta exact {rep['theta_exact']}/{n}", flush=True)
    return reports


def pick_tensors(inp, max_params=20_000_000):
    """Smallest, median-size and largest-affordable tensors of the call."""
    sizes = [(n, t) for t, (_, _, n) in enumerate(inp.tensors)]
    sizes.sort()
    picks = {sizes[0][1], sizes[len(sizes) // 2][1]}
    for n, t in reversed(sizes):
        if n <= max_params:
            picks.add(t)
            break
    return sorted(picks)


def fragment_ids(cfg, which):
    numel = [s.numel for s in cfg.tensors]
    frag, loads = dlc.dlc_fragment_plan(numel, cfg.n_fragments)
    order = sorted(range(cfg.n_fragments), key=lambda p: (loads[p], p))
    p = {"median": order[cfg.n_fragments // 2], "largest": order[-1], "smallest": order[0]}[which]
    return [t for t, f in enumerate(frag) if f == p], p


def test_c1_full():
    cfg = workloads.config("c1")
    inp = workloads.fragment_inputs(cfg, [0], DEV)
    theta, mom = inp.theta_g.clone(), inp.momentum.clone()
    codes, cb, rng = run_call(inp, theta, mom, cfg.lr, cfg.beta)
    check_sampled(inp, [0], inp.theta_g, inp.momentum, theta, mom, codes, cb, rng, cfg, "c1")


def test_c2_full_cycle_of_24_fragments():
    """135M set: every one of the 24 fragments merged in turn; sampled tensors from
    the median fragment and the embedding fragment checked against the oracle."""
    cfg = workloads.config("c2")
    ids = list(range(len(cfg.tensors)))
    inp = workloads.fragment_inputs(cfg, ids, DEV)
    numel = [s.numel for s in cfg.tensors]
    frag, loads = dlc.dlc_fragment_plan(numel, 24)
    theta, mom = inp.theta_g.clone(), inp.momentum.clone()
    outs = {}
    for p in range(24):
        sel = [t for t in ids if frag[t] == p]
        if not sel:
            continue
        sub = workloads.StepInputs(inp.theta_g, inp.momentum, inp.theta_L, [inp.tensors[t] for t in sel],
                                   inp.weights, inp.present, sel, inp.learner_stride)
        before = theta.clone()
        codes, cb, rng = run_call(sub, theta, mom, cfg.lr, cfg.beta)
        outs[p] = (sub, before, codes, cb, rng)
    order = sorted(range(24), key=lambda q: (loads[q], q))
    for p in (order[12], order[-1]):
        sub, before, codes, cb, rng = outs[p]
        # every tensor of this fragment was untouched before its own call
        check_sampled(sub, pick_tensors(sub), before, torch.zeros_like(mom), theta, mom, codes, cb, rng, cfg,
                      f"c2 fragment {p}")


def test_c3_ten_steps_with_momentum():
    """1B set, K=8, Dirichlet weights: 10 consecutive outer steps, fresh learners
    each step from the current theta, momentum carried; sampled tensors checked
    against the oracle at every step (inputs of step s are the GPU's state after
    step s - 1)."""
    cfg = workloads.config("c3")
    ids = list(range(len(cfg.tensors)))
    theta, mom, offs = workloads.build_global(cfg, ids, DEV)
    sig = workloads.tensor_sigmas(cfg, len(ids))
    w = workloads.base_weights(cfg)
    picks = None
    for step in range(10):
        theta_L, loffs, stride = workloads.build_learners(cfg, ids, theta, offs, DEV, step=step, sigmas=sig)
        tens = [(o, lo, cfg.tensors[t].numel) for o, lo, t in zip(offs, loffs, ids)]
        inp = workloads.StepInputs(theta, mom, theta_L, tens, w, [1] * cfg.n_learners, ids, stride)
        before_t, before_m = theta.clone(), mom.clone()
        codes, cb, rng = run_call(inp, theta, mom, cfg.lr, cfg.beta)
        if picks is None:
            picks = pick_tensors(inp, 12_000_000)
            largest = max(range(len(ids)), key=lambda t: (inp.tensors[t][2], -t))  # the 65.5M embedding
        if step in (0, 1, 9):
            check_sampled(inp, picks + ([largest] if step != 1 else []), before_t, before_m, theta, mom, codes, cb,
                          rng, cfg, f"c3 step {step}")
        del theta_L, codes
        torch.cuda.empty_cache()
    assert torch.isfinite(theta).all() and torch.isfinite(mom).all()


def test_c4_median_fragment():
    """10B set, K=14, outliers: the median fragment with its 14 replicas resident;
    sampled tensors up to a 58.7M-param MLP matrix against the full oracle."""
    cfg = workloads.config("c4")
    ids, p = fragment_ids(cfg, "median")
    inp = workloads.fragment_inputs(cfg, ids, DEV, fragment=p)
    theta, mom = inp.theta_g.clone(), inp.momentum.clone()
    codes, cb, rng = run_call(inp, theta, mom, cfg.lr, cfg.beta)
    check_sampled(inp, pick_tensors(inp, 60_000_000), inp.theta_g, inp.momentum, theta, mom, codes, cb, rng, cfg,
                  "c4 median")


CHUNK = 1 << 26
SAMPLES = 1 << 20


def test_c4_largest_fragment():
    """10B set: the largest fragment, one 525,336,576-param tensor (the embedding)
    with 14 learners, in the benchmark's call shape.  The full oracle over 7.4e9
    pseudo-gradient elements takes too long for a test, so the check uses what
    holds at any size, for every learner:
      * the range equals oracle.clip_range of the tensor's fp64 mean and population
        deviation, accumulated chunk by chunk on the host about a shift (within one
        fp32 ulp: the order of the fp64 sums differs);
      * codes at 2^20 sampled positions (random ones, both ends of the tensor) are
        bit-exact against oracle.encode with the GPU's (lo, wd);
      * every used codebook entry lies in its bucket, every empty one is its
        midpoint, the bucket counts sum to numel, and sum_c cb_c n_c equals the
        sum of the clipped values within the entries' rounding;
    and theta and momentum at the sampled positions are bit-exact against
    oracle.merge and oracle.nesterov on the GPU's codes and codebooks."""
    cfg = workloads.config("c4")
    ids, p = fragment_ids(cfg, "largest")
    assert len(ids) == 1
    inp = workloads.fragment_inputs(cfg, ids, DEV, fragment=p)
    off, loff, n = inp.tensors[0]
    k = inp.theta_L.shape[0]
    assert n == 525_336_576 and k == 14
    theta, mom = inp.theta_g.clone(), inp.momentum.clone()
    codes, cb, rng = run_call(inp, theta, mom, cfg.lr, cfg.beta)
    print(f"[c4 largest] GPU step done: {n} params x {k} learners", flush=True)
    rs = np.random.default_rng(11)
    idx = np.unique(np.concatenate([rs.integers(0, n, SAMPLES), np.arange(4096), np.arange(n - 5000, n)]))
    it = torch.from_numpy(idx).to(DEV)
    tg = inp.theta_g[off:off + n]
    w_hat = oracle.normalize_weights(inp.weights)
    sample_codes, sample_cbs = [], []
    for i in range(k):
        lo, hi, wd, _ = (np.float32(v) for v in parity.host(rng[i, 0]))
        shift = None
        s1 = s2 = xc_sum = 0.0
        counts = torch.zeros(256, dtype=torch.int64)
        for a in range(0, n, CHUNK):
            b = min(n, a + CHUNK)
            x = (tg[a:b] - inp.theta_L[i, loff + a:loff + b]).cpu()  # one IEEE fp32 subtraction
            if shift is None:
                shift = float(x[0])
            d = x.double() - shift
            s1 += float(d.sum())
            s2 += float((d * d).sum())
            xc_sum += float(x.clamp(float(lo), float(hi)).double().sum())
            counts += torch.bincount(codes[i, loff + a:loff + b].cpu(), minlength=256)
        mu = shift + s1 / n
        sigma = float(np.sqrt(max(s2 / n - (s1 / n) ** 2, 0.0)))
        want = oracle.clip_range(mu, sigma)
        for got, ref in zip((lo, hi, wd), want[:3]):
            assert parity.ulp_distance(np.array([got]), np.array([ref]))[0] <= 1, (i, got, ref)
        counts = counts.numpy()
        assert counts.sum() == n
        cbi = parity.host(cb[i, 0])
        cbd = cbi.astype(np.float64)
        c = np.arange(256)
        left = np.float64(lo) + c * np.float64(wd)
        right = left + np.float64(wd)
        right[255] = max(right[255], np.float64(hi))  # the last bucket also holds the values clipped to hi
        used = counts > 0
        slack = np.abs(np.spacing(cbi)).astype(np.float64) + np.float64(wd) * 2.0 ** -14
        assert np.all(cbd[used] >= left[used] - slack[used]) and np.all(cbd[used] <= right[used] + slack[used])
        mid = oracle.codebook(np.zeros(256), np.zeros(256, np.int64), lo, wd)
        np.testing.assert_array_equal(cbi[~used], mid[~used])
        tol = float(np.sum(counts * parity.codebook_bound(cbi, wd)))
        assert abs(float(np.sum(counts * cbd)) - xc_sum) <= tol, (i, float(np.sum(counts * cbd)), xc_sum, tol)
        xs = np.subtract(parity.host(tg[it]), parity.host(inp.theta_L[i, loff + it]), dtype=np.float32)
        cs = parity.host(codes[i, loff + it])
        np.testing.assert_array_equal(cs, oracle.encode(xs, lo, wd))
        sample_codes.append(cs)
        sample_cbs.append(cbi)
        print(f"[c4 largest] learner {i}: range within 1 ulp, {len(idx)} sampled codes bit-exact, "
              f"codebook invariants hold", flush=True)
    g = oracle.merge(sample_codes, sample_cbs, w_hat)
    th_o, mo_o = oracle.nesterov(parity.host(tg[it]), parity.host(inp.momentum[off + it]), g, cfg.lr, cfg.beta)
    np.testing.assert_array_equal(parity.host(theta[off + it]), th_o)
    np.testing.assert_array_equal(parity.host(mom[off + it]), mo_o)
    print(f"[c4 largest] theta and momentum bit-exact at {len(idx)} sampled positions", flush=True)


def test_c5_k1_whole_set():
    """3000-tensor edge mix, K=1, weight 1, one call over every tensor: constant
    tensors, 4096-vectors, 1024^2 and 4096x11008 matrices."""
    cfg = workloads.config("c5k1")
    ids = list(range(len(cfg.tensors)))
    inp = workloads.fragment_inputs(cfg, ids, DEV)
    theta, mom = inp.theta_g.clone(), inp.momentum.clone()
    codes, cb, rng = run_call(inp, theta, mom, cfg.lr, cfg.beta)
    picks = [0, 1999, 2000, 2899, 2900, 2990, 2991, 2999]
    check_sampled(inp, picks, inp.theta_g, inp.momentum, theta, mom, codes, cb, rng, cfg, "c5 k1")
    # K = 1, w = 1: g = cb[code] exactly (lr, beta as configured)
    for t in (2990, 2995):
        off, loff, n = inp.tensors[t]
        assert float(rng[0, t, 2]) == 0.0  # zero-variance tensor
        assert torch.all(codes[0, loff:loff + n] == 0)


def test_c5_k16_fragment_with_absent_learners():
    """Edge mix, K=16: a 347-tensor fragment where each learner is absent with
    probability 1/4 (weight 0, never read)."""
    cfg = workloads.config("c5k16")
    numel = [s.numel for s in cfg.tensors]
    frag, loads = dlc.dlc_fragment_plan(numel, 24)
    counts = [sum(1 for f in frag if f == p) for p in range(24)]
    p = max(range(24), key=lambda q: (counts[q], -q))
    ids = [t for t, f in enumerate(frag) if f == p]
    inp = workloads.fragment_inputs(cfg, ids, DEV, fragment=p)
    assert 0 < sum(inp.present) < 16
    # absent rows are poisoned: they must never be read
    for i, pr in enumerate(inp.present):
        if not pr:
            inp.theta_L[i].fill_(float("nan"))
    theta, mom = inp.theta_g.clone(), inp.momentum.clone()
    codes, cb, rng = run_call(inp, theta, mom, cfg.lr, cfg.beta)
    assert torch.isfinite(theta).all()
    picks = pick_tensors(inp, 46_000_000)  # up to a 4096 x 11008 matrix
    const = [j for j, t in enumerate(ids) if cfg.tensors[t].kind == "const"]
    check_sampled(inp, sorted(set(picks + const[:2])), inp.theta_g, inp.momentum, theta, mom, codes, cb, rng,
                  cfg, f"c5 k16 fragment {p}")


def test_c3_resume_from_a_checkpoint_is_bit_identical():
    """The library keeps no state between calls: the caller's theta and momentum
    are the whole outer-optimizer state.  Ten outer steps on the 1B set straight
    through equal five steps, a save and load of theta and momentum (through
    torch.save / torch.load with weights_only), and five more, bit for bit."""
    import io

    cfg = workloads.config("c3")
    ids = list(range(len(cfg.tensors)))
    sig = workloads.tensor_sigmas(cfg, len(ids))
    w = workloads.base_weights(cfg)

    def steps(theta, mom, offs, first, last):
        for step in range(first, last):
            theta_L, loffs, stride = workloads.build_learners(cfg, ids, theta, offs, DEV, step=step, sigmas=sig)
            tens = [(o, lo, cfg.tensors[t].numel) for o, lo, t in zip(offs, loffs, ids)]
            inp = workloads.StepInputs(theta, mom, theta_L, tens, w, [1] * cfg.n_learners, ids, stride)
            run_call(inp, theta, mom, cfg.lr, cfg.beta)
            del theta_L
            torch.cuda.empty_cache()

    theta_a, mom_a, offs = workloads.build_global(cfg, ids, DEV)
    steps(theta_a, mom_a, offs, 0, 10)
    print("[c3 resume] ten steps straight done", flush=True)
    theta_b, mom_b, _ = workloads.build_global(cfg, ids, DEV)
    steps(theta_b, mom_b, offs, 0, 5)
    buf = io.BytesIO()
    torch.save({"theta": theta_b.cpu(), "momentum": mom_b.cpu(), "step": 5}, buf)
    del theta_b, mom_b
    torch.cuda.empty_cache()
    buf.seek(0)
    ck = torch.load(buf, weights_only=True)
    assert ck["step"] == 5
    theta_b, mom_b = ck["theta"].to(DEV), ck["momentum"].to(DEV)
    steps(theta_b, mom_b, offs, 5, 10)
    print("[c3 resume] five steps, checkpoint, five steps done", flush=True)
    assert torch.equal(theta_a, theta_b) and torch.equal(mom_a, mom_b)
    assert not torch.equal(theta_a, workloads.build_global(cfg, ids, DEV)[0])


def test_c2_resume_mid_cycle_is_bit_identical():
    """The 135M set's 24-fragment cycle (dlc_outer_cycle, one stream) against the
    same cycle interrupted after fragment 11: theta, momentum and the fragment
    cursor saved and loaded (torch.save / torch.load with weights_only), then
    fragments 12..23 through dlc_quantize + dlc_merge_outer_step, bit for bit."""
    import io

    cfg = workloads.config("c2")
    ids = list(range(len(cfg.tensors)))
    inp = workloads.fragment_inputs(cfg, ids, DEV)
    k, stride = inp.theta_L.shape
    frag, _ = dlc.dlc_fragment_plan([s.numel for s in cfg.tensors], 24)
    tens, first, order = dlc.group_by_fragment(inp.tensors, frag, 24)
    w = [list(inp.weights) for _ in range(24)]
    codes, cb, rng = dlc.outputs_for(k, stride, len(tens), DEV)
    ws = torch.empty(max(256, dlc.dlc_cycle_workspace_bytes(k, tens, first)), dtype=torch.uint8, device=DEV)
    theta_a, mom_a = inp.theta_g.clone(), inp.momentum.clone()
    dlc.dlc_outer_cycle(theta_a, mom_a, inp.theta_L, tens, first, w, codes, cb, rng, ws, cfg.lr, cfg.beta)
    torch.cuda.synchronize()

    theta_b, mom_b = inp.theta_g.clone(), inp.momentum.clone()

    def fragments(theta, mom, lo, hi):
        for p in range(lo, hi):
            sel = tens[first[p]:first[p + 1]]
            if not sel:
                continue
            sub = workloads.StepInputs(theta, mom, inp.theta_L, sel, inp.weights, inp.present, [], stride)
            run_call(sub, theta, mom, cfg.lr, cfg.beta)

    fragments(theta_b, mom_b, 0, 12)
    buf = io.BytesIO()
    torch.save({"theta": theta_b.cpu(), "momentum": mom_b.cpu(), "next_fragment": 12}, buf)
    del theta_b, mom_b
    buf.seek(0)
    ck = torch.load(buf, weights_only=True)
    theta_b, mom_b = ck["theta"].to(DEV), ck["momentum"].to(DEV)
    fragments(theta_b, mom_b, ck["next_fragment"], 24)
    torch.cuda.synchronize()
    assert torch.equal(theta_a, theta_b) and torch.equal(mom_a, mom_b)
    assert not torch.equal(theta_a, inp.theta_g)


@pytest.mark.parametrize("key", ["c1", "c3", "c4_median", "c5k16"])
def test_full_size_calls_are_deterministic(key):
    """The benchmark's call shape twice on the same inputs: codes, codebooks,
    ranges, theta and momentum bit-identical (integer histograms and fixed-order
    reductions: no result depends on the order of atomics or of block completion)."""
    if key == "c4_median":
        cfg = workloads.config("c4")
        ids, p = fragment_ids(cfg, "median")
    elif key == "c5k16":
        cfg = workloads.config("c5k16")
        ids, p = fragment_ids(cfg, "median")
    else:
        cfg = workloads.config(key)
        ids, p = list(range(len(cfg.tensors))), 0
    inp = workloads.fragment_inputs(cfg, ids, DEV, fragment=p)
    outs = []
    for _ in range(2):
        theta, mom = inp.theta_g.clone(), inp.momentum.clone()
        codes, cb, rng = run_call(inp, theta, mom, cfg.lr, cfg.beta)
        outs.append((codes, cb, rng, theta, mom))
    (c0, b0, r0, t0, m0), (c1, b1, r1, t1, m1) = outs
    assert torch.equal(t0, t1) and torch.equal(m0, m1)
    assert torch.equal(b0[[i for i, q in enumerate(inp.present) if q]], b1[[i for i, q in enumerate(inp.present) if q]])
    assert torch.equal(r0[[i for i, q in enumerate(inp.present) if q]], r1[[i for i, q in enumerate(inp.present) if q]])
    for i, q in enumerate(inp.present):
        if q:
            for (_, lo, n) in inp.tensors:
                assert torch.equal(c0[i, lo:lo + n], c1[i, lo:lo + n])
