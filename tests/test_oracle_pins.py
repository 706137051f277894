"""Pins of the CPU oracle against what the pages and the mathematics fix.

Every test here runs on the CPU.  None retypes the oracle's formula: each checks
it against a printed value (the INTELLECT-1 worked example), a closed form, an
exact-rational brute force on tiny inputs, an invariant, or a textbook result.
"""
import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
F32 = np.float32


# --- exact-rational helpers (brute force, independent of numpy's float ops) ----

def rn32(q: Fraction) -> np.float32:
    """The fp32 value nearest to the rational q, ties to even mantissa."""
    c = np.float32(float(q))
    best = None
    for cand in (np.nextafter(c, F32(-np.inf)), c, np.nextafter(c, F32(np.inf))):
        if not np.isfinite(cand):
            continue
        d = abs(Fraction(float(cand)) - q)
        if best is None or d < best[0]:
            best = (d, cand)
        elif d == best[0]:
            mant = int(np.array(cand, F32).view(np.uint32)) & 1
            if mant == 0:
                best = (d, cand)
    return F32(best[1])


def exact_code(x, lo, wd) -> int:
    """Bucket index by exact rationals with explicit fp32 rounding of each step."""
    t = rn32(Fraction(float(x)) - Fraction(float(lo)))
    q = rn32(Fraction(float(t)) / Fraction(float(wd)))
    c = math.floor(Fraction(float(q)))
    return min(max(c, 0), 255)


# --- worked example (INTELLECT-1 notes, section 3.2) -------------------------

def test_worked_example_4096x4096():
    gold = json.load(open(os.path.join(GOLDEN, "worked_example.json")))
    cfg = workloads.config("c1")
    inp = workloads.fragment_inputs(cfg, [0], "cpu")
    n = inp.tensors[0][2]
    assert n == gold["shape"][0] * gold["shape"][1]
    x = oracle.pseudo_gradient(inp.theta_g[:n].numpy(), inp.theta_L[0, :n].numpy())
    q = oracle.quantize_tensor(x)
    # sampling bounds for n = 16.8M draws of N(0, sigma^2): 5 standard errors
    se_sigma = gold["sigma"] / math.sqrt(2 * n)
    se_mu = gold["sigma"] / math.sqrt(n)
    assert abs(q["mu"] - gold["mu"]) < 5 * se_mu
    assert abs(q["sigma"] - gold["sigma"]) < 5 * se_sigma
    assert abs(float(q["lo"]) - gold["clip_lo"]) < 5 * (se_mu + 6 * se_sigma)
    assert abs(float(q["hi"]) - gold["clip_hi"]) < 5 * (se_mu + 6 * se_sigma)
    # the printed width has two significant digits
    assert round(float(q["wd"]), 6) == pytest.approx(gold["bucket_width_printed"], abs=0.5e-6)
    # 256 buckets of width wd span the clip range
    assert float(q["wd"]) * gold["n_buckets"] == pytest.approx(float(q["hi"]) - float(q["lo"]), rel=1e-6)
    mb = 1 << 20
    assert x.nbytes == gold["bytes_fp32_MB"] * mb
    assert q["codes"].nbytes == gold["bytes_uint8_MB"] * mb
    assert x.nbytes // q["codes"].nbytes == gold["reduction"]
    # codes use the whole byte range and nearly nothing is clipped (~2e-9 * n)
    assert q["codes"].min() >= 0 and q["codes"].max() <= 255
    assert int(q["bucket_count"][0] + q["bucket_count"][255]) < 20


def test_worked_example_range_from_printed_sigma():
    """mu = 0, sigma = 1.2e-3 gives the printed range and width."""
    lo, hi, wd, m, deg = oracle.clip_range(0.0, 1.2e-3)
    assert not deg
    assert float(lo) == pytest.approx(-7.2e-3, rel=1e-7)
    assert float(hi) == pytest.approx(7.2e-3, rel=1e-7)
    assert float(wd) == pytest.approx(5.6e-5, abs=0.05e-5)
    assert float(wd) == pytest.approx(7.2e-3 * 2 / 256, rel=1e-7)


# --- statistics: closed forms and exact rationals ------------------------------

def test_stats_arithmetic_progression():
    a, h, n = 0.25, 2.0 ** -10, 1000
    x = (a + h * np.arange(n)).astype(F32)
    assert np.all(x.astype(np.float64) == a + h * np.arange(n))  # exactly representable
    mu, sigma = oracle.tensor_stats(x)
    assert mu == pytest.approx(a + (n - 1) * h / 2, rel=1e-15)
    assert sigma == pytest.approx(h * math.sqrt((n * n - 1) / 12.0), rel=1e-13)


def test_stats_two_point():
    x = np.array([-3e-3] * 500 + [5e-3] * 500, dtype=F32)
    mu, sigma = oracle.tensor_stats(x)
    a, b = float(F32(-3e-3)), float(F32(5e-3))
    assert mu == pytest.approx((a + b) / 2, rel=1e-14)
    assert sigma == pytest.approx(abs(b - a) / 2, rel=1e-14)


@pytest.mark.parametrize("seed", range(5))
def test_stats_exact_rational(seed):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal(37) * 1e-3 + 2e-4).astype(F32)
    fr = [Fraction(float(v)) for v in x]
    mu_e = sum(fr) / len(fr)
    var_e = sum((v - mu_e) ** 2 for v in fr) / len(fr)
    mu, sigma = oracle.tensor_stats(x)
    assert mu == pytest.approx(float(mu_e), rel=1e-14, abs=1e-19)
    assert sigma == pytest.approx(math.sqrt(float(var_e)), rel=1e-13)


# --- bucket index: exact grid, rational brute force, invariants ----------------

def test_encode_exact_grid_boundaries():
    lo, wd = F32(-1.0), F32(2.0 ** -7)   # lo + c*wd exact in fp32 for c = 0..256
    edges = np.array([float(lo) + c * float(wd) for c in range(256)], dtype=F32)
    assert np.all(oracle.encode(edges, lo, wd) == np.arange(256))
    below = np.nextafter(edges[1:], F32(-np.inf))
    # for x in [-1, -0.5] the subtraction x - lo is exact (Sterbenz) and the
    # division by a power of two is exact: one ulp below edge c lands in c - 1
    assert np.all(oracle.encode(below[:64], lo, wd) == np.arange(64))
    # elsewhere x - lo may round up onto the edge; the exact-rational rule decides
    assert list(oracle.encode(below, lo, wd)) == [exact_code(v, lo, wd) for v in below]
    # below the range -> 0, at and above lo + 256 wd -> 255
    out = oracle.encode(np.array([-5.0, np.nextafter(F32(-1), F32(-2)), 1.0, 1.5, 1e30], F32), lo, wd)
    assert list(out) == [0, 0, 255, 255, 255]


@pytest.mark.parametrize("seed", range(8))
def test_encode_rational_bruteforce(seed):
    rng = np.random.default_rng(100 + seed)
    sigma = float(10 ** rng.uniform(-5, -1))
    lo, hi, wd, _, deg = oracle.clip_range(float(rng.normal() * sigma), sigma)
    assert not deg
    x = (rng.standard_normal(64) * sigma * 3).astype(F32)
    # plant values on or next to bucket edges and beyond the clip range
    c = rng.integers(0, 256, 16)
    edge = (lo.astype(np.float64) + c * wd.astype(np.float64)).astype(F32)
    x = np.concatenate([x, edge, np.nextafter(edge, F32(np.inf)), np.nextafter(edge, F32(-np.inf)),
                        np.array([lo, hi, np.nextafter(lo, F32(-1)), np.nextafter(hi, F32(1))], F32)])
    got = oracle.encode(x, lo, wd)
    want = [exact_code(v, lo, wd) for v in x]
    assert list(got) == want


def test_encode_monotone_and_permutation():
    rng = np.random.default_rng(7)
    x = (rng.standard_normal(100_000) * 1e-3).astype(F32)
    q = oracle.quantize_tensor(x)
    order = np.argsort(x, kind="stable")
    assert np.all(np.diff(q["codes"][order].astype(np.int64)) >= 0)
    perm = rng.permutation(x.size)
    q2 = oracle.quantize_tensor(x[perm])
    assert np.array_equal(q2["codes"], q["codes"][perm])
    assert np.array_equal(q2["codebook"], q["codebook"]) or np.allclose(q2["codebook"], q["codebook"], rtol=1e-7)


@pytest.mark.parametrize("k", [-20, -3, 5])
def test_power_of_two_scaling(k):
    rng = np.random.default_rng(11)
    x = (rng.standard_normal(50_000) * 1e-3).astype(F32)
    s = F32(2.0 ** k)
    qa = oracle.quantize_tensor(x)
    qb = oracle.quantize_tensor((x * s).astype(F32))
    assert np.array_equal(qa["codes"], qb["codes"])
    assert qb["lo"] == qa["lo"] * s and qb["hi"] == qa["hi"] * s and qb["wd"] == qa["wd"] * s
    assert np.array_equal(qb["codebook"], (qa["codebook"] * s).astype(F32))


# --- histogram and codebook: rational brute force and the section 4.1 claims ---

@pytest.mark.parametrize("seed", range(4))
def test_histogram_and_codebook_bruteforce(seed):
    rng = np.random.default_rng(200 + seed)
    x = (rng.standard_normal(200) * 1e-3).astype(F32)
    x[:4] = [F32(0.05), F32(-0.05), F32(0.06), F32(-0.06)]   # force clipping at both ends
    q = oracle.quantize_tensor(x)
    lo, hi, wd = q["lo"], q["hi"], q["wd"]
    sums, counts = {}, {}
    for v in x:
        c = exact_code(v, lo, wd)
        vc = min(max(Fraction(float(v)), Fraction(float(lo))), Fraction(float(hi)))
        sums[c] = sums.get(c, Fraction(0)) + vc
        counts[c] = counts.get(c, 0) + 1
    for c in range(256):
        assert int(q["bucket_count"][c]) == counts.get(c, 0)
        if c in counts:
            assert q["bucket_sum"][c] == pytest.approx(float(sums[c]), rel=1e-15, abs=1e-300)
            mean = sums[c] / counts[c]
            assert abs(Fraction(float(q["codebook"][c])) - mean) <= abs(Fraction(float(np.spacing(q["codebook"][c]))))
        else:  # empty bucket -> its midpoint
            mid = Fraction(float(lo)) + (c + Fraction(1, 2)) * Fraction(float(wd))
            assert abs(Fraction(float(q["codebook"][c])) - mid) <= abs(Fraction(float(np.spacing(q["codebook"][c]))))
    assert sum(counts.values()) == x.size
    assert int(q["bucket_count"][0]) >= 2 and int(q["bucket_count"][255]) >= 2


def _tensors_for_invariants():
    rng = np.random.default_rng(5)
    gauss = (rng.standard_normal(1 << 20) * 1.2e-3).astype(F32)
    t4 = (rng.standard_t(4, 1 << 20) * (1e-3 / math.sqrt(2))).astype(F32)
    lap = rng.laplace(0, 7e-4, 1 << 18).astype(F32)
    return [("gauss", gauss), ("student_t4", t4), ("laplace", lap)]


@pytest.mark.parametrize("name,x", _tensors_for_invariants())
def test_codebook_invariants(name, x):
    q = oracle.quantize_tensor(x)
    xc = oracle.clip_values(x, q["lo"], q["hi"])
    codes, cb, n = q["codes"], q["codebook"], q["bucket_count"]
    # each entry lies between the smallest and largest clipped value of its bucket
    mins = np.full(256, np.inf)
    maxs = np.full(256, -np.inf)
    np.minimum.at(mins, codes, xc.astype(np.float64))
    np.maximum.at(maxs, codes, xc.astype(np.float64))
    used = n > 0
    assert np.all(cb[used] >= mins[used].astype(F32)) and np.all(cb[used] <= maxs[used].astype(F32))
    # ... hence inside its nominal bucket (up to one rounding of the index)
    lo, wd = float(q["lo"]), float(q["wd"])
    c = np.arange(256)
    assert np.all(cb[used] >= (lo + c[used] * wd) - 2 * wd * 2.0 ** -23 * 256)
    assert np.all(cb[used] <= (lo + (c[used] + 1) * wd) + abs(float(q["hi"]) - (lo + 256 * wd)) + 1e-12)
    # sum_c cb[c] n_c equals the clipped sum
    assert float(np.sum(cb.astype(np.float64) * n)) == pytest.approx(float(np.sum(xc.astype(np.float64))), rel=1e-6, abs=1e-12)
    # the mean codebook's squared error is no larger than the midpoint codebook's
    mid = (lo + (c + 0.5) * wd).astype(F32)
    mse_mean = np.mean((cb[codes].astype(np.float64) - xc) ** 2)
    mse_mid = np.mean((mid[codes].astype(np.float64) - xc) ** 2)
    assert mse_mean <= mse_mid
    if name == "gauss":
        assert mse_mean == pytest.approx(wd * wd / 12, rel=0.01)


def test_clip_rates_match_closed_forms():
    """Fraction clipped at 6 sigma: Gaussian 1.97e-9, Laplace exp(-6 sqrt 2)."""
    rng = np.random.default_rng(9)
    lap = rng.laplace(0, 7e-4, 1 << 22).astype(F32)
    q = oracle.quantize_tensor(lap)
    clipped = np.mean((lap < q["lo"]) | (lap > q["hi"]))
    assert clipped == pytest.approx(math.exp(-6 * math.sqrt(2)), rel=0.1)


def test_degenerate_constant_tensor():
    for c in (0.0, 3.25e-4, -1e-2):
        x = np.full(4096, c, dtype=F32)
        q = oracle.quantize_tensor(x)
        assert q["degenerate"]
        assert np.all(q["codes"] == 0)
        assert np.all(q["codebook"] == F32(c))
        assert np.array_equal(oracle.dequantize(q["codes"], q["codebook"]), x)


# --- merge: special cases and the FedAvg reduction ------------------------------

def _learners(k, n=20_000, seed=0, scale=1e-3):
    rng = np.random.default_rng(seed)
    tg = (rng.standard_normal(n) * 0.02).astype(F32)
    th = np.stack([(tg - (rng.standard_normal(n) * scale).astype(F32)).astype(F32) for _ in range(k)])
    return tg, th


def test_merge_single_learner_is_dequantized_delta():
    tg, th = _learners(1)
    x = oracle.pseudo_gradient(tg, th[0])
    q = oracle.quantize_tensor(x)
    g = oracle.merge([q["codes"]], [q["codebook"]], oracle.normalize_weights([1.0]))
    assert np.array_equal(g, q["codebook"][q["codes"]].astype(np.float64))


def test_merge_identical_learners():
    tg, th = _learners(1)
    q = oracle.quantize_tensor(oracle.pseudo_gradient(tg, th[0]))
    w = oracle.normalize_weights([1.0, 2.5, 1.5])  # raw weights, total 5
    g = oracle.merge([q["codes"]] * 3, [q["codebook"]] * 3, w)
    np.testing.assert_allclose(g, q["codebook"][q["codes"]], rtol=1e-15)


def test_merge_learner_permutation():
    tg, th = _learners(4, seed=3)
    qs = [oracle.quantize_tensor(oracle.pseudo_gradient(tg, th[i])) for i in range(4)]
    w = oracle.normalize_weights([0.1, 0.4, 0.2, 0.3])
    g1 = oracle.merge([q["codes"] for q in qs], [q["codebook"] for q in qs], w)
    p = [2, 0, 3, 1]
    g2 = oracle.merge([qs[i]["codes"] for i in p], [qs[i]["codebook"] for i in p], [w[i] for i in p])
    # reordering the fp64 sum changes only its last bits
    np.testing.assert_allclose(g1, g2, rtol=1e-14, atol=1e-15 * float(np.max(np.abs(g1))))


def test_fedavg_reduction_pins_the_sign():
    """lr = 1, beta = 0, v = 0: theta_new = theta_g - g ~ sum_i w_i theta_i, within
    the quantization error (at most one bucket width per learner when unclipped)."""
    tg, th = _learners(3, seed=4)
    w_raw = [1.0, 2.0, 1.0]
    w = oracle.normalize_weights(w_raw)
    tensors = [(0, 0, tg.size)]
    out = oracle.outer_step(tg, np.zeros_like(tg), th, tg.size, tensors, w_raw, lr=1.0, beta=0.0)
    avg = sum(wi * th[i].astype(np.float64) for i, wi in enumerate(w))
    bound = sum(wi * float(out["quant"][(i, 0)]["wd"]) for i, wi in enumerate(w)) + 4e-9
    unclipped = np.ones(tg.size, bool)
    for i in range(3):
        x = oracle.pseudo_gradient(tg, th[i])
        q = out["quant"][(i, 0)]
        unclipped &= (x >= q["lo"]) & (x <= q["hi"])
    err = np.abs(out["theta"].astype(np.float64) - avg)
    assert np.all(err[unclipped] <= bound)
    # the step moves theta toward the learners (wrong sign would double the distance)
    d_before = np.abs(tg.astype(np.float64) - avg).mean()
    assert np.abs(out["theta"] - avg).mean() < 0.2 * d_before


def test_adding_in_code_space_is_not_the_float_mean():
    """Section 4.2: Q(a) + Q(b) != Q(a + b).  Averaging codes instead of
    dequantized values gives a different merge."""
    tg, th = _learners(2, seed=8)
    qs = [oracle.quantize_tensor(oracle.pseudo_gradient(tg, th[i])) for i in range(2)]
    g = oracle.merge([q["codes"] for q in qs], [q["codebook"] for q in qs], [0.5, 0.5])
    code_avg = ((qs[0]["codes"].astype(np.int64) + qs[1]["codes"]) // 2).astype(np.uint8)
    wrong = qs[0]["codebook"][code_avg].astype(np.float64)
    assert np.mean(np.abs(wrong - g)) > 1e-2 * np.mean(np.abs(g))


def test_weights_and_quorum():
    assert oracle.normalize_weights([1, 1, 2]) == [0.25, 0.25, 0.5]
    with pytest.raises(oracle.NoQuorum):
        oracle.normalize_weights([0.0, 0.0])
    with pytest.raises(ValueError):
        oracle.normalize_weights([1.0, -1.0])
    tg, th = _learners(2)
    with pytest.raises(oracle.NoQuorum):
        oracle.outer_step(tg, np.zeros_like(tg), th, tg.size, [(0, 0, tg.size)], [0.0, 0.0])


def test_absent_learner_is_ignored():
    tg, th = _learners(3, seed=12)
    t = [(0, 0, tg.size)]
    a = oracle.outer_step(tg, np.zeros_like(tg), th, tg.size, t, [1.0, 0.0, 1.0])
    th2 = th.copy()
    th2[1] = np.nan  # an absent learner's bytes are never read
    b = oracle.outer_step(tg, np.zeros_like(tg), th2, tg.size, t, [1.0, 0.0, 1.0])
    assert np.array_equal(a["theta"], b["theta"]) and np.array_equal(a["momentum"], b["momentum"])


# --- Nesterov: closed form and torch.optim.SGD ----------------------------------

def test_nesterov_closed_form_constant_g():
    lr, beta = 0.7, 0.9
    g = np.array([1e-3, -2.5e-4, 3e-2, 0.0], np.float64)
    th0 = np.array([0.01, -0.02, 0.5, 1.0], F32)
    th, v = th0.copy(), np.zeros(4, F32)
    for t in range(1, 11):
        th, v = oracle.nesterov(th, v, g, lr, beta)
        v_cf = g * (1 - beta ** t) / (1 - beta)
        s = t + beta / (1 - beta) * (t - beta * (1 - beta ** t) / (1 - beta))
        th_cf = th0.astype(np.float64) - lr * g * s
        np.testing.assert_allclose(v, v_cf, rtol=1e-6, atol=1e-12)
        np.testing.assert_allclose(th, th_cf, rtol=1e-6, atol=1e-9)
    # printed special cases: t = 1 -> 1.9 lr g, t = 2 -> 4.61 lr g
    assert 1 + beta / (1 - beta) * (1 - beta * (1 - beta) / (1 - beta)) == pytest.approx(1.9)
    assert 2 + beta / (1 - beta) * (2 - beta * (1 - beta ** 2) / (1 - beta)) == pytest.approx(4.61)


def test_nesterov_matches_torch_sgd():
    """One torch.optim.SGD(nesterov=True) step per outer step, started from the
    oracle's fp32 state each time: the oracle equals torch's fp64 result rounded
    to fp32 (within one fp32 ulp)."""
    rng = np.random.default_rng(21)
    th = (rng.standard_normal(1000) * 0.02).astype(F32)
    v = np.zeros_like(th)
    for step in range(5):
        g = rng.standard_normal(1000) * 1e-3
        p = torch.nn.Parameter(torch.tensor(th.astype(np.float64)))
        opt = torch.optim.SGD([p], lr=0.7, momentum=0.9, nesterov=True)
        if step > 0:
            opt.state[p]["momentum_buffer"] = torch.tensor(v.astype(np.float64))
        p.grad = torch.tensor(g)
        opt.step()
        th, v = oracle.nesterov(th, v, g)
        th_t = p.detach().numpy()
        v_t = opt.state[p]["momentum_buffer"].numpy()
        assert np.all(np.abs(th - th_t) <= np.abs(np.spacing(th)))
        assert np.all(np.abs(v - v_t) <= np.abs(np.spacing(v)))


# --- fragment plan: hand-worked case, brute-force optimum, textbook bound -------

def test_lpt_hand_worked():
    # 7 -> f0; 5 -> f1; 4 -> f1 (5 < 7); 3 -> f0 (7 < 9); 3 -> f1 (9 < 10); 2 -> f0 (10 < 12)
    frag, loads = oracle.fragment_plan([7, 5, 4, 3, 3, 2], 2)
    assert frag == [0, 1, 1, 0, 1, 0] and loads == [12, 12]
    # ties between equal sizes go to the lower tensor index first
    frag, loads = oracle.fragment_plan([3, 3, 3], 2)
    assert frag == [0, 1, 0] and loads == [6, 3]
    # more fragments than tensors leaves fragments empty
    frag, loads = oracle.fragment_plan([5, 1], 4)
    assert frag == [0, 1] and loads == [5, 1, 0, 0]


@pytest.mark.parametrize("seed", range(20))
def test_lpt_graham_bound(seed):
    rng = np.random.default_rng(seed)
    t = int(rng.integers(1, 9))
    p = int(rng.integers(1, 4))
    sizes = [int(v) for v in rng.integers(1, 100, t)]
    frag, loads = oracle.fragment_plan(sizes, p)
    assert sorted(set(frag)) <= list(range(p)) and len(frag) == t
    assert sum(loads) == sum(sizes)
    for q in range(p):
        assert loads[q] == sum(s for s, f in zip(sizes, frag) if f == q)
    opt = min(max(sum(s for s, f in zip(sizes, a) if f == q) for q in range(p))
              for a in itertools.product(range(p), repeat=t))
    assert max(loads) <= (Fraction(4, 3) - Fraction(1, 3 * p)) * opt


def test_lpt_on_model_sets():
    for key in ("c2", "c4", "c5k1"):
        cfg = workloads.config(key)
        numel = [s.numel for s in cfg.tensors]
        frag, loads = oracle.fragment_plan(numel, 24)
        assert sum(loads) == sum(numel)
        # no fragment exceeds the largest tensor or the mean load by more than one tensor
        assert max(loads) <= max(max(numel), sum(numel) / 24 + max(numel))


# --- whole-call invariants ---------------------------------------------------------

def _small_model_inputs():
    cfg = workloads.config("c2")
    ids = [1, 2, 3, 4, 5, 6]  # attn_norm, q, k, v, o, mlp_norm of layer 0
    return cfg, workloads.fragment_inputs(cfg, ids, "cpu")


def test_fragmenting_does_not_change_the_result():
    """One call over all tensors equals one call per fragment (tensors are independent)."""
    cfg, inp = _small_model_inputs()
    tg, mom, tl = inp.theta_g.numpy(), inp.momentum.numpy(), inp.theta_L.numpy()
    whole = oracle.outer_step(tg, mom, tl, inp.learner_stride, inp.tensors, inp.weights)
    frag, _ = oracle.fragment_plan([n for _, _, n in inp.tensors], 3)
    th, v = tg.copy(), mom.copy()
    for p in (2, 0, 1):  # any visiting order
        sel = [t for t, f in zip(inp.tensors, frag) if f == p]
        before = th.copy()
        out = oracle.outer_step(th, v, tl, inp.learner_stride, sel, inp.weights)
        outside = np.ones(th.size, bool)
        for off, _, n in sel:
            outside[off:off + n] = False
        assert np.array_equal(out["theta"][outside], before[outside])
        th, v = out["theta"], out["momentum"]
    assert np.array_equal(th, whole["theta"]) and np.array_equal(v, whole["momentum"])


def test_workload_parameter_counts():
    counts = {k: sum(s.numel for s in workloads.config(k).tensors) for k in ("c2", "c3", "c4", "c5k1")}
    # 135M tied: 30 layers x (2*576 + 2*576^2 + 2*192*576 + 3*576*1536) + 49152*576 + 576
    assert counts["c2"] == 30 * (2 * 576 + 2 * 576 ** 2 + 2 * 192 * 576 + 3 * 576 * 1536) + 49152 * 576 + 576
    assert counts["c3"] == 16 * (2 * 2048 + 2 * 2048 ** 2 + 2 * 512 * 2048 + 3 * 2048 * 5632) + 2 * 32000 * 2048 + 2048
    assert counts["c4"] == 42 * (2 * 4096 + 2 * 4096 ** 2 + 2 * 1024 * 4096 + 3 * 4096 * 14336) + 2 * 128256 * 4096 + 4096
    assert counts["c5k1"] == 2000 * 4096 + 900 * 1024 ** 2 + 90 * 4096 * 11008 + 10 * 4096
    assert len(workloads.config("c2").tensors) == 272
    assert len(workloads.config("c3").tensors) == 147
    assert len(workloads.config("c4").tensors) == 381


# ---------------------------------------------------------------------------
# The fragment cycle and sending the update back (Decoupled DiLoCo digest,
# "architecture"; INTELLECT-1 notes, section 3.2 step 8).
# ---------------------------------------------------------------------------
def _cycle_case(seed=0, sizes=(700, 64 * 40 + 3, 4096, 100, 2048), k=3):
    rng = np.random.default_rng(seed)
    offs, pos = [], 0
    for n in sizes:
        offs.append(pos)
        pos += (n + 63) // 64 * 64
    theta = (rng.standard_normal(pos) * 0.02).astype(np.float32)
    mom = (rng.standard_normal(pos) * 1e-3).astype(np.float32)
    tl = np.zeros((k, pos), np.float32)
    for i in range(k):
        tl[i] = (theta - rng.standard_normal(pos) * 1e-3).astype(np.float32)
    tensors = [(o, o, n) for o, n in zip(offs, sizes)]
    return theta, mom, tl, pos, tensors


def test_broadcast_copies_exactly_and_only_the_tensors():
    theta, _, tl, stride, tensors = _cycle_case()
    out = oracle.broadcast(theta, tl, tensors[1:3], rows=[1, 0, 1])
    for i in range(3):
        for t, (o, lo, n) in enumerate(tensors):
            if t in (1, 2) and i != 1:
                np.testing.assert_array_equal(out[i, lo:lo + n], theta[o:o + n])
            else:
                np.testing.assert_array_equal(out[i, lo:lo + n], tl[i, lo:lo + n])


def test_cycle_with_one_fragment_is_outer_step():
    theta, mom, tl, stride, tensors = _cycle_case(1)
    w = [0.2, 0.5, 0.3]
    cyc = oracle.outer_cycle(theta, mom, tl, stride, tensors, [0, len(tensors)], [w])
    one = oracle.outer_step(theta, mom, tl, stride, tensors, w)
    np.testing.assert_array_equal(cyc["theta"], one["theta"])
    np.testing.assert_array_equal(cyc["momentum"], one["momentum"])


def test_cycle_result_does_not_depend_on_fragment_order():
    theta, mom, tl, stride, tensors = _cycle_case(2)
    w = [[1.0, 1.0, 0.0], [0.3, 0.3, 0.4], [1.0, 0.0, 0.0]]
    a = oracle.outer_cycle(theta, mom, tl, stride, tensors, [0, 2, 3, 5], w, send_back=True)
    # the same fragments, listed in reverse order
    rev = tensors[3:5] + tensors[2:3] + tensors[0:2]
    b = oracle.outer_cycle(theta, mom, tl, stride, rev, [0, 2, 3, 5], w[::-1], send_back=True)
    for key in ("theta", "momentum", "theta_L"):
        np.testing.assert_array_equal(a[key], b[key])


def test_rda_cycle_is_its_fragments_rda_steps_stitched():
    # Without send-back nothing couples disjoint fragments: the cycle equals each
    # fragment's own RDA step from the initial state, stitched together.
    theta, mom, tl, stride, tensors = _cycle_case(4)
    w = [[1.0, 2.0, 0.5], [0.0, 1.0, 3.0], [2.0, 2.0, 2.0]]
    first = [0, 2, 3, 5]
    cyc = oracle.outer_cycle(theta, mom, tl, stride, tensors, first, w, rule="rda")
    th, mo = theta.copy(), mom.copy()
    for f in range(3):
        sel = tensors[first[f]:first[f + 1]]
        one = oracle.outer_step(theta, mom, tl, stride, sel, w[f], [1 if x > 0 else 0 for x in w[f]], rule="rda")
        for o, _, n in sel:
            th[o:o + n] = one["theta"][o:o + n]
            mo[o:o + n] = one["momentum"][o:o + n]
    np.testing.assert_array_equal(cyc["theta"], th)
    np.testing.assert_array_equal(cyc["momentum"], mo)


def test_rda_cycle_is_not_the_mean_cycle():
    # learners of very different norms: averaging directions and norms separately
    # moves theta differently from the weighted mean
    theta, mom, tl, stride, tensors = _cycle_case(5)
    tl[2] = theta - 10.0 * (theta - tl[2])
    w = [[1.0, 1.0, 1.0], [1.0, 2.0, 1.0]]
    first = [0, 3, 5]
    a = oracle.outer_cycle(theta, mom, tl, stride, tensors, first, w, rule="rda")
    b = oracle.outer_cycle(theta, mom, tl, stride, tensors, first, w)
    assert np.max(np.abs(a["theta"] - b["theta"])) > 1e-4


def test_after_sending_back_the_next_cycle_is_a_pure_momentum_step():
    # Once every learner holds the merged theta, each pseudo-gradient is exactly
    # zero: every tensor is degenerate (codes 0, codebook = mean = 0), g = 0, and
    # Nesterov reduces to v <- beta v, theta <- theta - lr beta^2 v.
    theta, mom, tl, stride, tensors = _cycle_case(3)
    w = [[1.0, 2.0, 3.0], [1.0, 1.0, 1.0]]
    first = [0, 3, 5]
    c1 = oracle.outer_cycle(theta, mom, tl, stride, tensors, first, w, send_back=True)
    c2 = oracle.outer_cycle(c1["theta"], c1["momentum"], c1["theta_L"], stride, tensors, first, w)
    lr, beta = 0.7, 0.9
    for o, _, n in tensors:
        v = c1["momentum"][o:o + n].astype(np.float64)
        t = c1["theta"][o:o + n].astype(np.float64)
        np.testing.assert_array_equal(c2["momentum"][o:o + n], (beta * v).astype(np.float32))
        np.testing.assert_array_equal(c2["theta"][o:o + n], (t - lr * (beta * (beta * v))).astype(np.float32))
    for f, res in c2["steps"].items():
        for q in res["quant"].values():
            assert q["degenerate"] and not q["codes"].any()


# ---------------------------------------------------------------------------
# Learners reporting against older bases (Decoupled DiLoCo digest, "fault
# tolerance": asynchronous learners).
# ---------------------------------------------------------------------------
def test_bases_equal_to_theta_g_change_nothing():
    theta, mom, tl, stride, tensors = _cycle_case(4)
    w = [0.5, 0.3, 0.2]
    a = oracle.outer_step(theta, mom, tl, stride, tensors, w)
    b = oracle.outer_step(theta, mom, tl, stride, tensors, w, bases=[theta, theta.copy(), theta.copy()])
    np.testing.assert_array_equal(a["theta"], b["theta"])
    np.testing.assert_array_equal(a["momentum"], b["momentum"])


def test_stale_learner_without_progress_only_dilutes_the_others():
    # Learner 2 reports against an old base it never moved away from: its
    # pseudo-gradient is exactly zero, its codebook all zeros, so the merged
    # g equals the other learners' merge scaled by W / (W + w_2).
    theta, mom, tl, stride, tensors = _cycle_case(5)
    rng = np.random.default_rng(9)
    old = (theta + rng.standard_normal(theta.shape) * 1e-3).astype(np.float32)
    tl = tl.copy()
    tl[2] = old
    w = [1.0, 3.0, 2.0]
    with_stale = oracle.outer_step(theta, mom, tl, stride, tensors, w, bases=[theta, theta, old])
    without = oracle.outer_step(theta, mom, tl, stride, tensors, [1.0, 3.0, 0.0])
    for t in with_stale["g"]:
        assert with_stale["quant"][(2, t)]["degenerate"]
        # fp64 sums of the same terms with different weights: a few ulps of the
        # largest term, relative where g does not cancel
        scale = float(np.abs(without["g"][t]).max())
        np.testing.assert_allclose(with_stale["g"][t], without["g"][t] * (4.0 / 6.0), rtol=1e-13, atol=1e-15 * scale)


# ---------------------------------------------------------------------------
# The ring with requantization at every hop (INTELLECT-1 notes, section 3.2
# step 6 and section 4.2).
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("n", [1, 63, 64, 65, 100, 1000, 4096 * 3 + 17])
@pytest.mark.parametrize("k", [1, 2, 3, 8, 14])
def test_ring_chunks_tile_the_tensor(n, k):
    ch = oracle.ring_chunks(n, k)
    assert len(ch) == k and ch[0][0] == 0 and ch[-1][1] == n
    for (a, b), (c, d) in zip(ch, ch[1:]):
        assert b == c and a <= b
    for a, b in ch[:-1]:
        assert a % 64 == 0 and b % 64 == 0
    sizes = [b - a for a, b in ch]
    assert max(sizes) - min(s for s in sizes) <= 64 + n % 64 or n < 64 * k


def test_ring_with_one_rank_is_the_star_merge():
    theta, mom, tl, stride, tensors = _cycle_case(6, k=1)
    ring = oracle.ring_outer_step(theta, mom, tl, stride, tensors)
    star = oracle.outer_step(theta, mom, tl, stride, tensors, [1.0])
    np.testing.assert_array_equal(ring["theta"], star["theta"])
    np.testing.assert_array_equal(ring["momentum"], star["momentum"])


@pytest.mark.parametrize("k", [2, 3, 5])
def test_ring_on_constant_chunks_is_the_ring_order_fp32_mean(k):
    # Every message of a constant chunk has zero variance, so quantization is
    # lossless; chunk c's sum is then Delta_c + Delta_{c+1} + ... + Delta_{c-1}
    # added left to right in fp32 (the order the ring visits the ranks), and the
    # mean fl32(sum / k).
    n = 64 * 7 + 5
    rng = np.random.default_rng(k)
    theta = np.full(n, 1.0, np.float32)
    ch = oracle.ring_chunks(n, k)
    consts = rng.uniform(-1e-3, 1e-3, (k, k)).astype(np.float32)  # [rank, chunk]
    tl = np.zeros((k, n + 64), np.float32)
    for r in range(k):
        for c, (a, b) in enumerate(ch):
            tl[r, a:b] = np.float32(1.0) - consts[r, c]
    delta = np.array([[np.float32(1.0) - tl[r, ch[c][0]] for c in range(k)] for r in range(k)], np.float32)
    res = oracle.ring_outer_step(theta, np.zeros(n, np.float32), tl, n + 64, [(0, 0, n)])
    for c, (a, b) in enumerate(ch):
        if b == a:
            continue
        s = np.float32(0.0)
        for j in range(k):
            s = np.float32(s + delta[(c + j) % k, c]) if j else delta[c, c]
        want = np.float32(s / np.float32(k))
        np.testing.assert_array_equal(res["g"][0][a:b], np.full(b - a, want, np.float32))


def test_ring_error_exceeds_the_star_and_grows_with_the_ring():
    # Requantizing a running sum at every hop adds quantization noise each time;
    # a star merge quantizes each pseudo-gradient once, so its error averages down
    # as 1/sqrt(K) while the ring's does not: the ratio grows with K.
    n = 64 * 2000
    rng = np.random.default_rng(1)
    theta = (rng.standard_normal(n) * 0.02).astype(np.float32)
    errs = {}
    for k in (2, 8):
        tl = np.stack([(theta - rng.standard_normal(n) * 1e-3).astype(np.float32) for _ in range(k)])
        exact = np.mean([theta.astype(np.float64) - tl[r].astype(np.float32).astype(np.float64) for r in range(k)], 0)
        mom = np.zeros(n, np.float32)
        ring = oracle.ring_outer_step(theta, mom, tl, n, [(0, 0, n)])
        star = oracle.outer_step(theta, mom, tl, n, [(0, 0, n)], [1.0] * k)
        e_ring = float(np.sqrt(np.mean((ring["g"][0] - exact) ** 2)))
        e_star = float(np.sqrt(np.mean((star["g"][0] - exact) ** 2)))
        assert e_ring > e_star
        errs[k] = e_ring / e_star
    assert errs[8] > 1.5 * errs[2]


# ---------------------------------------------------------------------------
# Radial-Directional Averaging (Decoupled DiLoCo digest, "architecture", second
# engineering detail): directions and norms averaged separately.  The page gives
# no formula; these pins fix the reading g = (sum w_i ||x_i||) d / ||d||,
# d = sum w_i x_i / ||x_i||, through properties that hold for it and fail for
# the plausible slips (a plain mean, an unnormalized direction, unweighted
# norms).
# ---------------------------------------------------------------------------
def _rda_learners(k, n=5000, seed=0):
    rng = np.random.default_rng(seed)
    codes, cbs, xs = [], [], []
    for i in range(k):
        x = (rng.standard_normal(n) * 10.0 ** rng.uniform(-4, -2) + rng.uniform(-1e-4, 1e-4)).astype(np.float32)
        q = oracle.quantize_tensor(x)
        codes.append(q["codes"])
        cbs.append(q["codebook"])
        xs.append(oracle.dequantize(q["codes"], q["codebook"]).astype(np.float64))
    return codes, cbs, xs


def _halves(n, first, second):
    """codes / codebook of a vector equal to `first` on the first half, `second` on the rest."""
    codes = np.zeros(n, np.uint8)
    codes[: n // 2] = 1
    cb = np.zeros(256, np.float32)
    cb[0], cb[1] = second, first
    return codes, cb


def test_rda_one_learner_is_the_dequantized_delta():
    codes, cbs, xs = _rda_learners(1)
    np.testing.assert_allclose(oracle.rda_merge(codes, cbs, [1.0]), xs[0], rtol=1e-14, atol=0)


def test_rda_identical_learners():
    codes, cbs, xs = _rda_learners(1, seed=3)
    g = oracle.rda_merge(codes * 3, cbs * 3, oracle.normalize_weights([1.0, 5.0, 0.5]))
    np.testing.assert_allclose(g, xs[0], rtol=1e-14, atol=0)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_rda_norm_is_the_weighted_mean_norm(seed):
    codes, cbs, xs = _rda_learners(4, seed=seed)
    w = oracle.normalize_weights([1.0, 3.0, 0.25, 2.0])
    g = oracle.rda_merge(codes, cbs, w)
    want = sum(wi * np.linalg.norm(x) for wi, x in zip(w, xs))
    assert abs(np.linalg.norm(g) - want) <= 1e-12 * want


def test_rda_two_equal_weights_bisect_the_angle():
    codes, cbs, xs = _rda_learners(2, seed=5)
    n0, n1 = np.linalg.norm(xs[0]), np.linalg.norm(xs[1])
    assert max(n0, n1) > 2 * min(n0, n1)  # norms far apart, so a plain mean would not bisect
    g = oracle.rda_merge(codes, cbs, [0.5, 0.5])
    cos = [float(g @ x) / (np.linalg.norm(g) * np.linalg.norm(x)) for x in xs]
    assert abs(cos[0] - cos[1]) <= 1e-12
    # the plain mean leans toward the longer vector (the pin tells them apart)
    mean = 0.5 * (xs[0] + xs[1])
    cm = [float(mean @ x) / (np.linalg.norm(mean) * np.linalg.norm(x)) for x in xs]
    assert abs(cm[0] - cm[1]) > 1e-3


@pytest.mark.parametrize("a,b", [(3.0, 1.0), (-2.0, 0.5), (0.25, -4.0)])
def test_rda_orthogonal_halves_closed_form(a, b):
    # x1 = a on the first half, x2 = b on the second: the directions are
    # orthogonal, ||d|| = 1/sqrt(2), and g = (|a| + |b|) / (2 sqrt(2)) times the
    # signs, where the plain mean would give a/2 and b/2.
    n = 1000
    c1, cb1 = _halves(n, np.float32(a), np.float32(0.0))
    c2, cb2 = _halves(n, np.float32(0.0), np.float32(b))
    g = oracle.rda_merge([c1, c2], [cb1, cb2], [0.5, 0.5])
    mag = (abs(a) + abs(b)) / (2.0 * math.sqrt(2.0))
    np.testing.assert_allclose(g[: n // 2], np.sign(a) * mag, rtol=1e-15)
    np.testing.assert_allclose(g[n // 2:], np.sign(b) * mag, rtol=1e-15)


def test_rda_opposite_learners_cancel():
    codes, cbs, xs = _rda_learners(1, seed=7)
    neg = [np.negative(cbs[0])]
    g = oracle.rda_merge(codes * 2, cbs + neg, [0.5, 0.5])
    assert np.all(g == 0.0)


def _rda_constants(values, n=5000):
    """codes / codebooks of learners whose dequantized tensors are the given constants."""
    codes, cbs = [], []
    for v in values:
        q = oracle.quantize_tensor(np.full(n, np.float32(v), np.float32))
        codes.append(q["codes"])
        cbs.append(q["codebook"])
    return codes, cbs


@pytest.mark.parametrize("seed", [2, 3, 4, 5])
def test_rda_balanced_constant_learners_give_zero(seed):
    # Twelve learners moved a tensor by constants, six up and six down, under equal
    # weights: every u_i is +-1/sqrt(n) times the same vector, so d = 0 exactly in
    # real arithmetic and g = 0.  (In fp64, with n not a power of two, the norms
    # round and d keeps ~1e-16 of noise, which an exact-zero test would normalize
    # into a full-size step.)
    rng = np.random.default_rng(seed)
    signs = np.array([1.0] * 6 + [-1.0] * 6)
    rng.shuffle(signs)
    codes, cbs = _rda_constants(signs * 10.0 ** rng.uniform(-5, -3, 12))
    g = oracle.rda_merge(codes, cbs, [1.0 / 12] * 12)
    assert np.all(g == 0.0)


@pytest.mark.parametrize("eps", [1e-3, 1e-6])
def test_rda_nearly_opposite_constants_closed_form(eps):
    # x1 = c1, x2 = -c2 (constants) with weights 1/2 + eps and 1/2 - eps: d = 2 eps
    # times the unit vector of ones, so g = w1 c1 + w2 c2 on every element (the
    # averaged norm along the heavier learner's direction), however small eps is
    # as long as d is more than rounding noise.
    c1, c2 = 3e-4, 7e-4
    codes, cbs = _rda_constants([c1, -c2])
    w1, w2 = 0.5 + eps, 0.5 - eps
    g = oracle.rda_merge(codes, cbs, [w1, w2])
    x1, x2 = float(np.float32(c1)), float(np.float32(c2))
    np.testing.assert_allclose(g, w1 * x1 + w2 * x2, rtol=1e-12)


def test_rda_zero_learner_adds_no_direction():
    # r = w1 r1 and d = w1 u1, so g = w1 x1: a learner that did not move dilutes
    # the norm by its weight and nothing else.
    codes, cbs, xs = _rda_learners(1, seed=8)
    z = oracle.quantize_tensor(np.zeros(len(codes[0]), np.float32))
    w = oracle.normalize_weights([3.0, 1.0])
    g = oracle.rda_merge([codes[0], z["codes"]], [cbs[0], z["codebook"]], w)
    np.testing.assert_allclose(g, 0.75 * xs[0], rtol=1e-14)


def test_rda_scaling_one_learner_changes_only_the_norm():
    codes, cbs, xs = _rda_learners(3, seed=9)
    w = oracle.normalize_weights([1.0, 2.0, 1.5])
    g = oracle.rda_merge(codes, cbs, w)
    cbs4 = [cbs[0], (cbs[1] * np.float32(4.0)).astype(np.float32), cbs[2]]
    g4 = oracle.rda_merge(codes, cbs4, w)
    np.testing.assert_allclose(g4 / np.linalg.norm(g4), g / np.linalg.norm(g), rtol=1e-12, atol=1e-15)
    grow = np.linalg.norm(g4) - np.linalg.norm(g)
    assert abs(grow - w[1] * 3.0 * np.linalg.norm(xs[1])) <= 1e-12 * np.linalg.norm(g4)


def test_rda_outer_step_with_one_learner_is_the_star_step():
    theta, mom, tl, stride, tensors = _cycle_case(12, k=1)
    a = oracle.outer_step(theta, mom, tl, stride, tensors, [1.0], rule="rda")
    b = oracle.outer_step(theta, mom, tl, stride, tensors, [1.0])
    for t in range(len(tensors)):
        np.testing.assert_allclose(a["g"][t], b["g"][t], rtol=1e-14, atol=0)
    np.testing.assert_allclose(a["theta"], b["theta"], rtol=2 ** -23, atol=0)


@pytest.mark.parametrize("bad", [np.nan, np.inf, -np.inf])
def test_non_finite_pseudo_gradients_are_refused(bad):
    x = np.zeros(100, np.float32)
    x[37] = bad
    with pytest.raises(ValueError):
        oracle.quantize_tensor(x)
