"""GPU tests of the ring with requantization at every hop (dlc_ring_outer_step)
against the CPU oracle's ring_outer_step.

* one rank: bit-identical to the star path (dlc_quantize + a one-learner merge);
* constant chunks (every message lossless): bit-identical to the oracle,
  including the fp32 ring-order sums and the division by K;
* the 1B set at K = 8, every tensor in one call, sampled tensors against the
  oracle with the bar below;
* Gaussian pseudo-gradients (K up to 16): the GPU's codebooks may differ from
  the oracle's by an ulp, which can move a later hop's code to the neighbouring
  bucket; that chunk's later sums, ranges and codes then differ too (the ring
  requantizes what it received).  The bar: per chunk, either 99.9% of theta
  within 1e-9 + 1e-5 |theta| or the chunk counts as diverged; no more chunks
  diverge than measured on the committed seeds (none up to K = 8, two of 48 at
  K = 16, one of 24 on the 1B set's sampled tensors); every diverged chunk matches
  the oracle's messages up to a hop whose codes differ by adjacent-bucket flips
  only; every element within the bucket widths the messages can shift it by; the GPU's g within 5% (RMS) of the
  exact mean's scale from the oracle's g; and every gather message of a chunk
  that has not diverged has the oracle's range within one ulp and, where the
  range is identical, its codes (up to a 1e-3 share of adjacent-bucket flips
  from sums an earlier flip moved).
"""
import numpy as np
import pytest
import torch

import diloco_outer_step_amd as dlc
import oracle
import workloads
from tests import parity

pytestmark = pytest.mark.gpu

DEV = "cuda"
LR, BETA = 0.7, 0.9


def packed(sizes):
    offs, pos = [], 0
    for n in sizes:
        offs.append(pos)
        pos += (n + 63) // 64 * 64
    return [(o, o, n) for o, n in zip(offs, sizes)], pos


def gpu_ring(theta, mom, theta_L, tensors, messages=False):
    th, mo = theta.clone(), mom.clone()
    accum, codes, cb, rng = dlc.ring_buffers(theta_L, len(tensors))
    ws = torch.empty(max(256, dlc.dlc_ring_workspace_bytes(theta_L.shape[0], tensors)), dtype=torch.uint8,
                     device=DEV)
    dlc.dlc_ring_outer_step(th, mo, theta_L, tensors, accum, codes, cb, rng, ws, LR, BETA)
    torch.cuda.synchronize()
    if messages:
        return th, mo, codes, rng
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


def check_against_oracle(th_g, orc, theta, theta_L, tensors, k, t_ids=None):
    """The ring parity bar, per tensor (o, lo, n) of `tensors` (GPU and oracle
    results at the same offsets): returns (diverged chunks, chunks).  t_ids: the
    oracle's tensor index of each entry (default: its position)."""
    th_g, th_o = th_g.astype(np.float64), orc["theta"].astype(np.float64)
    diverged = chunks = 0
    check_against_oracle.diverged = set()  # (entry j, chunk start) of every diverged chunk
    for j, (o, lo, n) in enumerate(tensors):
        t = j if t_ids is None else t_ids[j]
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
                check_against_oracle.diverged.add((j, a))
            assert d.max() <= LR * (1 + BETA) * 2.0 * wd, f"tensor {t} chunk [{a}, {b}): max |dtheta| {d.max():.3e}"
        # both rings are equally far from the exact mean of the pseudo-gradients
        exact = np.mean([theta[o:o + n].astype(np.float64) - theta_L[r, lo:lo + n].astype(np.float64)
                         for r in range(k)], 0)
        ref = theta[o:o + n].astype(np.float64)
        g_gpu = (ref - th_g[o:o + n]) / LR  # g + beta v_new, same v for both
        g_orc = (ref - th_o[o:o + n]) / LR
        e_gpu = np.sqrt(np.mean((g_gpu - g_orc) ** 2))
        assert e_gpu <= 0.05 * np.sqrt(np.mean(exact ** 2))
    return diverged, chunks


def check_gather_messages(codes, rng, orc, tensors, k, diverged):
    """The gather messages the GPU returns (one range row per non-empty owned chunk,
    tensor by tensor, rank by rank; codes in each owner's row at the chunk) against
    the oracle's hop K - 1 messages, on every chunk that has not diverged: the range
    within one fp32 ulp (its statistics are the ones the last dequantize-add formed),
    the codes bit-exact where the range is bit-identical.  Returns the number of
    gather messages checked."""
    codes, rng = host(codes), host(rng)
    gather = [(t, r, c, q) for (t, s, r, c, q) in orc["messages"] if s == k - 1]
    checked = 0
    for row, (t, r, c, q) in enumerate(gather):
        a, b = oracle.ring_chunks(tensors[t][2], k)[c]
        if (t, a) in diverged:
            continue
        ro = np.array([q["lo"], q["hi"], q["wd"]], np.float32)
        d = parity.ulp_distance(rng[row, :3], ro)
        assert d.max() <= 1, f"tensor {t} rank {r} chunk [{a}, {b}): gather range {rng[row, :3]} vs {ro}"
        if d.max() == 0:
            # a chunk that has not diverged may still hold a few sums an earlier flip moved
            lo = tensors[t][1]
            got = codes[r, lo + a:lo + b].astype(np.int64)
            mism = got != q["codes"]
            assert mism.mean() <= 1e-3, f"tensor {t} chunk [{a}, {b}): {int(mism.sum())} gather codes differ"
            assert np.all(np.abs(got[mism] - q["codes"][mism].astype(np.int64)) <= 1)
        checked += 1
    return checked


def check_divergence_origins(codes, orc, tensors, k, diverged):
    """Where each diverged chunk left the oracle's ring.  Every hop's messages
    survive in the code buffer (sender r writes chunk (r - s) mod K at stage s, a
    different chunk at every stage), so the chunk's messages can be compared hop by
    hop: the first one whose codes differ must differ only by adjacent-bucket
    flips, on at most a 1e-3 share of the chunk -- a code on the other side of a
    bucket edge that an ulp of difference in a range or a sum moved -- and every
    earlier hop must match exactly.  Returns the first differing hop per chunk."""
    codes = host(codes)
    msg = {(t, s, c): (r, q) for (t, s, r, c, q) in orc["messages"]}
    first = {}
    for j, a in sorted(diverged):
        _, lo, n = tensors[j]
        chunks = oracle.ring_chunks(n, k)
        c = next(i for i, (x, y) in enumerate(chunks) if x == a and y > x)
        b = chunks[c][1]
        for s in range(k):
            r, q = msg[(j, s, c)]
            got = codes[r, lo + a:lo + b].astype(np.int64)
            want = q["codes"].astype(np.int64)
            mism = got != want
            if mism.any():
                assert np.all(np.abs(got[mism] - want[mism]) == 1), f"tensor {j} chunk [{a}, {b}) hop {s}"
                assert mism.mean() <= 1e-3, f"tensor {j} chunk [{a}, {b}) hop {s}: {int(mism.sum())} codes differ"
                first[(j, a)] = (s, int(mism.sum()))
                break
        else:
            raise AssertionError(f"tensor {j} chunk [{a}, {b}) diverged with every message's codes equal")
    return first


# diverged chunks measured on these seeds with the current kernels: none up to
# K = 8, two of 48 at K = 16
MAX_DIVERGED = {2: 0, 4: 0, 8: 0, 16: 2}


@pytest.mark.parametrize("k", [2, 4, 8, 16])
def test_gaussian_against_oracle(k):
    sizes = [64 * 300 + 9, 4096 * 8, 50000]
    tensors, stride = packed(sizes)
    g = torch.Generator(device=DEV)
    g.manual_seed(10 + k)
    theta = torch.randn(stride, generator=g, device=DEV) * 0.02
    mom = torch.randn(stride, generator=g, device=DEV) * 1e-3
    theta_L = torch.stack([theta - torch.randn(stride, generator=g, device=DEV) * 1e-3 for _ in range(k)])
    th, mo, codes, rng = gpu_ring(theta, mom, theta_L, tensors, messages=True)
    orc = oracle.ring_outer_step(host(theta), host(mom), host(theta_L), stride, tensors, LR, BETA)
    diverged, chunks = check_against_oracle(host(th), orc, host(theta), host(theta_L), tensors, k)
    print(f"[ring K = {k}] {diverged} of {chunks} chunks diverged", flush=True)
    assert diverged <= MAX_DIVERGED[k], f"{diverged} of {chunks} chunks diverged"
    origins = check_divergence_origins(codes, orc, tensors, k, check_against_oracle.diverged)
    print(f"[ring K = {k}] first differing hop and codes per diverged chunk: {origins}", flush=True)
    checked = check_gather_messages(codes, rng, orc, tensors, k, check_against_oracle.diverged)
    assert checked == chunks - diverged


@pytest.mark.slow
def test_ring_full_1b_set_sampled_tensors():
    """The ring over all 147 tensors of the 1B set at K = 8, in the launch layout
    the bench times; sampled tensors against the oracle's ring over those tensors
    alone (every message is one chunk of one tensor, so tensors are independent)."""
    cfg = workloads.config("c3")
    inp = workloads.fragment_inputs(cfg, list(range(len(cfg.tensors))), DEV)
    k = inp.theta_L.shape[0]
    theta0, mom0 = inp.theta_g.clone(), inp.momentum.clone()
    th, mo, codes, _ = gpu_ring(inp.theta_g, inp.momentum, inp.theta_L, inp.tensors, messages=True)
    sizes = sorted((n, t) for t, (_, _, n) in enumerate(inp.tensors))
    # the smallest tensor, the largest below 2M and the largest below 5M elements (2048, 512 x 2048, 2048^2)
    picks = sorted({sizes[0][1], max((n, t) for n, t in sizes if n <= 2_000_000)[1],
                    max((n, t) for n, t in sizes if n <= 5_000_000)[1]})
    sub, stride = packed([inp.tensors[t][2] for t in picks])
    th0 = np.zeros(stride, np.float32)
    mo0 = np.zeros(stride, np.float32)
    tl = np.zeros((k, stride), np.float32)
    th_gpu = np.zeros(stride, np.float32)
    for (o2, _, n), t in zip(sub, picks):
        o, lo, _ = inp.tensors[t]
        th0[o2:o2 + n] = host(theta0[o:o + n])
        mo0[o2:o2 + n] = host(mom0[o:o + n])
        tl[:, o2:o2 + n] = host(inp.theta_L[:, lo:lo + n])
        th_gpu[o2:o2 + n] = host(th[o:o + n])
    orc = oracle.ring_outer_step(th0, mo0, tl, stride, sub, LR, BETA)
    diverged, chunks = check_against_oracle(th_gpu, orc, th0, tl, sub, k)
    # the picked tensors where the GPU's code buffer holds them
    at_gpu = [(inp.tensors[t][0], inp.tensors[t][1], n) for (_, _, n), t in zip(sub, picks)]
    origins = check_divergence_origins(codes, orc, at_gpu, k, check_against_oracle.diverged)
    print(f"[ring c3] tensors {picks} ({[n for _, _, n in sub]} params, K = {k}): "
          f"{diverged} of {chunks} chunks diverged, first differing hops {origins}", flush=True)
    assert diverged <= 1  # measured: one of 24
