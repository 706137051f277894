"""GPU tests of sending the update back (dlc_broadcast) and of a whole outer step
over every fragment with overlapped streams (dlc_outer_cycle).

* broadcast: bit-exact copies, for every padded row count the kernel is built
  for (4, 8, 12, 16 rows) and the run-time row count, ragged tails, row subsets;
* cycle: bit-exact against the same calls made fragment by fragment, on one and
  on two streams, on two lanes, and through dlc_outer_cycle_lanes on 1, 3 and 4
  lanes; against the oracle's cycle with the parity bar of tests/parity.py; the
  135M set's 24-fragment cycle with send-back.
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
RAGGED = [1, 63, 64, 65, 577, 4095, 4096, 4097, 12289, 100003]


def packed(sizes):
    offs, pos = [], 0
    for n in sizes:
        offs.append(pos)
        pos += (n + 63) // 64 * 64
    return [(o, o, n) for o, n in zip(offs, sizes)], pos


@pytest.mark.parametrize("k", [1, 3, 8, 12, 16, 20])
def test_broadcast_bit_exact(k):
    tensors, stride = packed(RAGGED + [4096 * 9 + 5])
    g = torch.Generator(device=DEV)
    g.manual_seed(100 + k)
    theta = torch.randn(stride, generator=g, device=DEV)
    theta_L = torch.randn((k, stride), generator=g, device=DEV)
    before = theta_L.clone()
    rows = [1 if (i % 3) != 1 else 0 for i in range(k)] if k > 1 else None
    sel = tensors[1::2]  # every other tensor: the others must stay untouched
    dlc.dlc_broadcast(theta, theta_L, sel, rows=rows)
    torch.cuda.synchronize()
    want = oracle.broadcast(theta.cpu().numpy(), before.cpu().numpy(), sel, rows)
    np.testing.assert_array_equal(theta_L.cpu().numpy(), want)


def cycle_inputs(seed, k, sizes, n_fragments, absent=True):
    """Random theta, momentum, replicas; fragments from the greedy plan, grouped."""
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    tensors, stride = packed(sizes)
    theta = torch.randn(stride, generator=g, device=DEV) * 0.02
    mom = torch.randn(stride, generator=g, device=DEV) * 1e-3
    theta_L = (theta - torch.randn((k, stride), generator=g, device=DEV) * 1e-3).contiguous()
    frag, _ = dlc.dlc_fragment_plan(sizes, n_fragments)
    grouped, first, _ = dlc.group_by_fragment(tensors, frag, n_fragments)
    rng = np.random.default_rng(seed)
    weights = []
    for f in range(n_fragments):
        w = rng.uniform(0.5, 2.0, k)
        if absent and k > 1:
            w[rng.random(k) < 0.3] = 0.0
            if not (w > 0).any():
                w[0] = 1.0
        weights.append([float(x) for x in w])
    return theta, mom, theta_L, grouped, first, weights


def run_cycle(theta, mom, theta_L, grouped, first, weights, broadcast, two_streams, two_lanes=False, lanes=None):
    """lanes: a list of streams (None = the current stream) for dlc_outer_cycle_lanes."""
    k, stride = theta_L.shape
    theta, mom, theta_L = theta.clone(), mom.clone(), theta_L.clone()
    codes, cb, rng = dlc.outputs_for(k, stride, len(grouped), DEV)
    copies = len(lanes) if lanes is not None else 2 if two_lanes else 1
    need = dlc.dlc_cycle_workspace_bytes(k, grouped, first) * copies
    ws = torch.empty(max(256, need), dtype=torch.uint8, device=DEV)
    qs = torch.cuda.current_stream()
    if lanes is not None:
        dlc.dlc_outer_cycle_lanes(theta, mom, theta_L, grouped, first, weights, codes, cb, rng, ws,
                                  [qs if s is None else s for s in lanes], broadcast=broadcast)
    else:
        ms = torch.cuda.Stream() if two_streams else qs
        dlc.dlc_outer_cycle(theta, mom, theta_L, grouped, first, weights, codes, cb, rng, ws, broadcast=broadcast,
                            quantize_stream=qs, merge_stream=ms, two_lanes=two_lanes)
    torch.cuda.synchronize()
    return dict(theta=theta, momentum=mom, theta_L=theta_L, codes=codes, codebook=cb, range=rng)


def run_sequential(theta, mom, theta_L, grouped, first, weights, broadcast):
    k, stride = theta_L.shape
    theta, mom, theta_L = theta.clone(), mom.clone(), theta_L.clone()
    codes, cb, rng = dlc.outputs_for(k, stride, len(grouped), DEV)
    for f in range(len(first) - 1):
        sel = grouped[first[f]:first[f + 1]]
        if not sel:
            continue
        present = [1 if w > 0 else 0 for w in weights[f]]
        _, cbf, rf = dlc.outputs_for(k, 64, len(sel), DEV)
        ws = dlc.alloc_workspace(k, sel, DEV)
        dlc.dlc_quantize(theta, theta_L, sel, codes, cbf, rf, ws, present=present)
        dlc.dlc_merge_outer_step(theta, mom, codes, cbf, weights[f], sel)
        if broadcast:
            dlc.dlc_broadcast(theta, theta_L, sel)
        torch.cuda.synchronize()
        for i in range(k):
            if present[i]:
                cb[i, first[f]:first[f + 1]] = cbf[i]
                rng[i, first[f]:first[f + 1]] = rf[i]
    return dict(theta=theta, momentum=mom, theta_L=theta_L, codes=codes, codebook=cb, range=rng)


def assert_same(a, b, weights, grouped, first):
    for key in ("theta", "momentum", "theta_L"):
        assert torch.equal(a[key], b[key]), key
    for f in range(len(first) - 1):
        for i, w in enumerate(weights[f]):
            if w <= 0:
                continue
            for t in range(first[f], first[f + 1]):
                _, lo, n = grouped[t]
                assert torch.equal(a["codes"][i, lo:lo + n], b["codes"][i, lo:lo + n])
                assert torch.equal(a["codebook"][i, t], b["codebook"][i, t])
                assert torch.equal(a["range"][i, t], b["range"][i, t])


@pytest.mark.parametrize("two_streams,two_lanes", [(False, False), (True, False), (True, True), (False, True)])
@pytest.mark.parametrize("broadcast", [False, True])
def test_cycle_equals_fragment_by_fragment(two_streams, two_lanes, broadcast):
    sizes = RAGGED + [4096] * 12 + [64 * 3000 + 7] * 3 + [1 << 18]
    args = cycle_inputs(7, 5, sizes, 7)
    a = run_cycle(*args, broadcast=broadcast, two_streams=two_streams, two_lanes=two_lanes)
    b = run_sequential(*args, broadcast=broadcast)
    assert_same(a, b, args[5], args[3], args[4])


@pytest.mark.parametrize("n_lanes,repeat", [(1, False), (3, False), (4, False), (3, True)])
@pytest.mark.parametrize("broadcast", [False, True])
def test_lanes_equal_fragment_by_fragment(n_lanes, repeat, broadcast):
    """dlc_outer_cycle_lanes on 1, 3 and 4 streams, and on three lanes of which two
    share a stream."""
    sizes = RAGGED + [4096] * 12 + [64 * 3000 + 7] * 3 + [1 << 18]
    args = cycle_inputs(9, 4, sizes, 9)
    streams = [None] + [torch.cuda.Stream() for _ in range(n_lanes - 1)]
    if repeat:
        streams[2] = streams[1]
    a = run_cycle(*args, broadcast=broadcast, two_streams=False, lanes=streams)
    b = run_sequential(*args, broadcast=broadcast)
    assert_same(a, b, args[5], args[3], args[4])


def test_cycle_against_oracle_with_empty_fragment_and_absent_learners():
    sizes = [5000, 4096 * 3 + 1, 777, 64 * 100, 9000]
    theta, mom, theta_L, grouped, first, weights = cycle_inputs(11, 4, sizes, 7)  # 7 > 5 tensors: empty fragments
    assert any(first[f] == first[f + 1] for f in range(7))
    gpu = run_cycle(theta, mom, theta_L, grouped, first, weights, broadcast=True, two_streams=True)
    k, stride = theta_L.shape
    orc = oracle.outer_cycle(theta.cpu().numpy(), mom.cpu().numpy(), theta_L.cpu().numpy(), stride, grouped, first,
                             weights, send_back=True)
    # per fragment, the parity bar of a single call (each fragment's tensors only)
    for f, res in orc["steps"].items():
        sel = grouped[first[f]:first[f + 1]]
        view = workloads.StepInputs(theta, mom, theta_L, sel, weights[f], [1 if w > 0 else 0 for w in weights[f]],
                                    list(range(len(sel))), stride)
        g = dict(codes=gpu["codes"], codebook=gpu["codebook"][:, first[f]:first[f + 1]],
                 range=gpu["range"][:, first[f]:first[f + 1]], theta=gpu["theta"], momentum=gpu["momentum"])
        parity.compare(g, res, view, pinned=False)
    # sending back: every learner row holds the GPU's own merged theta
    for _, lo, n in grouped:
        for i in range(k):
            assert torch.equal(gpu["theta_L"][i, lo:lo + n], gpu["theta"][lo:lo + n])


@pytest.mark.slow
def test_c2_cycle_with_send_back_equals_sequential():
    cfg = workloads.config("c2")
    ids = list(range(len(cfg.tensors)))
    inp = workloads.fragment_inputs(cfg, ids, DEV)
    frag, _ = dlc.dlc_fragment_plan([s.numel for s in cfg.tensors], 24)
    grouped, first, _ = dlc.group_by_fragment(inp.tensors, frag, 24)
    weights = [list(inp.weights)] * 24
    args = (inp.theta_g, inp.momentum, inp.theta_L, grouped, first, weights)
    a = run_cycle(*args, broadcast=True, two_streams=True)
    b = run_sequential(*args, broadcast=True)
    assert_same(a, b, weights, grouped, first)
    c = run_cycle(*args, broadcast=True, two_streams=True, two_lanes=True)
    assert_same(c, b, weights, grouped, first)
    d = run_cycle(*args, broadcast=True, two_streams=False, lanes=[None, torch.cuda.Stream(), torch.cuda.Stream()])
    assert_same(d, b, weights, grouped, first)


def run_cycle_rda(theta, mom, theta_L, grouped, first, weights, broadcast, lanes):
    """dlc_outer_cycle_rda on the given lanes (None = the current stream)."""
    k, stride = theta_L.shape
    theta, mom, theta_L = theta.clone(), mom.clone(), theta_L.clone()
    codes, cb, rng = dlc.outputs_for(k, stride, len(grouped), DEV)
    norms = torch.zeros((k, len(grouped)), dtype=torch.float64, device=DEV)
    need = (dlc.dlc_cycle_rda_workspace_bytes(k, grouped, first) + 256) * len(lanes)
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    qs = torch.cuda.current_stream()
    dlc.dlc_outer_cycle_rda(theta, mom, theta_L, grouped, first, weights, codes, cb, rng, norms, ws,
                            [qs if s is None else s for s in lanes], broadcast=broadcast)
    torch.cuda.synchronize()
    return dict(theta=theta, momentum=mom, theta_L=theta_L, codes=codes, codebook=cb, range=rng, sq_norms=norms)


def run_sequential_rda(theta, mom, theta_L, grouped, first, weights, broadcast):
    """dlc_rda_outer_step fragment by fragment on one stream."""
    k, stride = theta_L.shape
    theta, mom, theta_L = theta.clone(), mom.clone(), theta_L.clone()
    codes, cb, rng = dlc.outputs_for(k, stride, len(grouped), DEV)
    norms = torch.zeros((k, len(grouped)), dtype=torch.float64, device=DEV)
    for f in range(len(first) - 1):
        sel = grouped[first[f]:first[f + 1]]
        if not sel:
            continue
        _, cbf, rf = dlc.outputs_for(k, 64, len(sel), DEV)
        nf = torch.zeros((k, len(sel)), dtype=torch.float64, device=DEV)
        ws = torch.empty(max(256, dlc.dlc_rda_workspace_bytes(k, sel)), dtype=torch.uint8, device=DEV)
        dlc.dlc_rda_outer_step(theta, mom, theta_L, sel, weights[f], codes, cbf, rf, nf, ws)
        if broadcast:
            dlc.dlc_broadcast(theta, theta_L, sel)
        torch.cuda.synchronize()
        for i in range(k):
            if weights[f][i] > 0:
                cb[i, first[f]:first[f + 1]] = cbf[i]
                rng[i, first[f]:first[f + 1]] = rf[i]
                norms[i, first[f]:first[f + 1]] = nf[i]
    return dict(theta=theta, momentum=mom, theta_L=theta_L, codes=codes, codebook=cb, range=rng, sq_norms=norms)


@pytest.mark.parametrize("n_lanes", [1, 3, 4])
@pytest.mark.parametrize("broadcast", [False, True])
def test_rda_cycle_equals_fragment_by_fragment(n_lanes, broadcast):
    """dlc_outer_cycle_rda against dlc_rda_outer_step called fragment by fragment:
    the same kernels on the same partitions, so every output is bit-identical,
    the squared norms included."""
    sizes = RAGGED + [4096] * 12 + [64 * 3000 + 7] * 3 + [1 << 18]
    args = cycle_inputs(11, 5, sizes, 8)
    lanes = [None] + [torch.cuda.Stream() for _ in range(n_lanes - 1)]
    a = run_cycle_rda(*args, broadcast=broadcast, lanes=lanes)
    b = run_sequential_rda(*args, broadcast=broadcast)
    weights, grouped, first = args[5], args[3], args[4]
    assert_same(a, b, weights, grouped, first)
    for f in range(len(first) - 1):
        for i, w in enumerate(weights[f]):
            if w > 0:
                assert torch.equal(a["sq_norms"][i, first[f]:first[f + 1]], b["sq_norms"][i, first[f]:first[f + 1]])


def test_rda_cycle_against_oracle():
    """The RDA cycle with send-back, an empty fragment and absent learners against
    the oracle's cycle with the RDA rule: each fragment's quantization at the
    parity bar, and theta and momentum within the step tolerance wherever no code
    flipped."""
    sizes = [5000, 4096 * 3 + 1, 777, 64 * 100, 9000, 20000]
    k = 4
    theta, mom, theta_L, grouped, first, weights = cycle_inputs(13, k, sizes, 4)
    first = [0, 2, 2, 4, 6]  # fragment 1 empty
    stride = theta_L.shape[1]
    gpu = run_cycle_rda(theta, mom, theta_L, grouped, first, weights, broadcast=True,
                        lanes=[None, torch.cuda.Stream()])
    orc = oracle.outer_cycle(theta.cpu().numpy(), mom.cpu().numpy(), theta_L.cpu().numpy(), stride, grouped, first,
                             weights, send_back=True, rule="rda")
    th_g, th_o = parity.host(gpu["theta"]).astype(np.float64), orc["theta"].astype(np.float64)
    for f, res in orc["steps"].items():
        sel = grouped[first[f]:first[f + 1]]
        view = workloads.StepInputs(theta, mom, theta_L, sel, weights[f], [1 if w > 0 else 0 for w in weights[f]],
                                    list(range(len(sel))), stride)
        g = dict(codes=gpu["codes"], codebook=gpu["codebook"][:, first[f]:first[f + 1]],
                 range=gpu["range"][:, first[f]:first[f + 1]], theta=gpu["theta"], momentum=gpu["momentum"])
        rep = parity.compare(g, res, view, pinned=False, state=False)
        if rep["flips"] == 0:
            for o, _, n in sel:
                d = np.abs(th_g[o:o + n] - th_o[o:o + n])
                assert np.all(d <= parity.ATOL + parity.RTOL * np.abs(th_o[o:o + n])), (f, o)
    for _, lo, n in grouped:
        for i in range(k):
            assert torch.equal(gpu["theta_L"][i, lo:lo + n], gpu["theta"][lo:lo + n])
