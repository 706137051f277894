"""The calls of one outer step captured in a HIP graph (torch.cuda.graph) and
replayed: nothing in them allocates, waits or clears memory through the
runtime, so the captured launches replay bit for bit what an eager step does.
Each replay restarts from the same state, with the program's own eager work and
synchronizations between replays, and is checked against the eager result."""
import pytest
import torch

import diloco_outer_step_amd as dlc
import workloads

pytestmark = pytest.mark.gpu

DEV = "cuda"


def test_captured_step_replays_the_eager_step():
    sizes = [1, 65, 4097, 64 * 300 + 9, 100003]
    cfg = workloads.custom("graph", sizes, 3, weights="dirichlet")
    inp = workloads.fragment_inputs(cfg, list(range(len(sizes))), DEV)
    k, stride = inp.theta_L.shape
    # eager reference
    codes_e, cb_e, rng_e = dlc.outputs_for(k, stride, len(sizes), DEV)
    ws_e = dlc.alloc_workspace(k, inp.tensors, DEV)
    th_e, mo_e = inp.theta_g.clone(), inp.momentum.clone()
    dlc.dlc_quantize(th_e, inp.theta_L, inp.tensors, codes_e, cb_e, rng_e, ws_e)
    dlc.dlc_merge_outer_step(th_e, mo_e, codes_e, cb_e, inp.weights, inp.tensors)
    torch.cuda.synchronize()
    # static buffers for the graph
    codes, cb, rng = dlc.outputs_for(k, stride, len(sizes), DEV)
    ws = dlc.alloc_workspace(k, inp.tensors, DEV)
    th, mo = inp.theta_g.clone(), inp.momentum.clone()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            dlc.dlc_quantize(th, inp.theta_L, inp.tensors, codes, cb, rng, ws)
            dlc.dlc_merge_outer_step(th, mo, codes, cb, inp.weights, inp.tensors)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for rep in range(4):
        th.copy_(inp.theta_g)
        mo.copy_(inp.momentum)
        noise = torch.randn(1 << 20, device=DEV).sum()  # unrelated eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.isfinite(noise)
        for _, lo, n in inp.tensors:
            assert torch.equal(codes[:, lo:lo + n], codes_e[:, lo:lo + n]), rep
        assert torch.equal(cb, cb_e) and torch.equal(rng, rng_e), rep
        assert torch.equal(th, th_e) and torch.equal(mo, mo_e), rep


@pytest.mark.parametrize("mode", ["two_streams", "two_lanes", "three_lanes", "four_lanes", "rda_four_lanes"])
def test_captured_cycle_replays_the_eager_cycle(mode):
    """A whole fragment cycle on two streams (the second joins the capture through
    the cycle's own events), on two lanes, on three and four lanes through
    dlc_outer_cycle_lanes, and on four lanes merged by Radial-Directional
    Averaging (dlc_outer_cycle_rda), captured once and replayed."""
    two_lanes = mode == "two_lanes"
    rda = mode.startswith("rda")
    n_lanes = {"three_lanes": 3, "four_lanes": 4, "rda_four_lanes": 4}.get(mode, 0)
    sizes = [4096] * 6 + [64 * 1000 + 5] * 3 + [1 << 17, 777]
    cfg = workloads.custom("graph_cycle", sizes, 4)
    inp = workloads.fragment_inputs(cfg, list(range(len(sizes))), DEV)
    k, stride = inp.theta_L.shape
    frag, _ = dlc.dlc_fragment_plan(sizes, 5)
    grouped, first, _ = dlc.group_by_fragment(inp.tensors, frag, 5)
    weights = [list(inp.weights)] * 5
    need = (max(dlc.dlc_cycle_workspace_bytes(k, grouped, first), dlc.dlc_cycle_rda_workspace_bytes(k, grouped, first))
            + 256) * 4

    norms = {}  # sq_norms of each buffer set (RDA), by the codes buffer's address

    def buffers():
        codes, cb, rng = dlc.outputs_for(k, stride, len(grouped), DEV)
        norms[codes.data_ptr()] = torch.zeros((k, len(grouped)), dtype=torch.float64, device=DEV)
        ws = torch.empty(need, dtype=torch.uint8, device=DEV)
        return codes, cb, rng, ws, inp.theta_g.clone(), inp.momentum.clone(), inp.theta_L.clone()

    codes_e, cb_e, rng_e, ws_e, th_e, mo_e, tl_e = buffers()

    def cycle(th, mo, tl, codes, cb, rng, ws, first_stream, others):
        if rda:
            dlc.dlc_outer_cycle_rda(th, mo, tl, grouped, first, weights, codes, cb, rng, norms[codes.data_ptr()], ws,
                                    [first_stream] + others[:n_lanes - 1], broadcast=True)
        elif n_lanes:
            dlc.dlc_outer_cycle_lanes(th, mo, tl, grouped, first, weights, codes, cb, rng, ws,
                                      [first_stream] + others[:n_lanes - 1], broadcast=True)
        else:
            dlc.dlc_outer_cycle(th, mo, tl, grouped, first, weights, codes, cb, rng, ws, broadcast=True,
                                quantize_stream=first_stream, merge_stream=others[0], two_lanes=two_lanes)

    cycle(th_e, mo_e, tl_e, codes_e, cb_e, rng_e, ws_e, torch.cuda.current_stream(),
          [torch.cuda.Stream() for _ in range(3)])
    torch.cuda.synchronize()

    codes, cb, rng, ws, th, mo, tl = buffers()
    graph = torch.cuda.CUDAGraph()
    side, others = torch.cuda.Stream(), [torch.cuda.Stream() for _ in range(3)]
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            cycle(th, mo, tl, codes, cb, rng, ws, side, others)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for rep in range(3):
        th.copy_(inp.theta_g)
        mo.copy_(inp.momentum)
        tl.copy_(inp.theta_L)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(th, th_e) and torch.equal(mo, mo_e) and torch.equal(tl, tl_e), rep
        assert torch.equal(cb, cb_e) and torch.equal(rng, rng_e), rep
        if rda:
            assert torch.equal(norms[codes.data_ptr()], norms[codes_e.data_ptr()]), rep


@pytest.mark.parametrize("call", ["rda", "ring"])
def test_captured_rda_and_ring_replay_the_eager_calls(call):
    """dlc_rda_outer_step and dlc_ring_outer_step (several kernels each, ranges,
    codebooks, squared norms or ring messages in between) captured once and
    replayed: every replay equals the eager call bit for bit."""
    sizes = [1, 65, 4097, 64 * 300 + 9, 100003]
    cfg = workloads.custom("graph_" + call, sizes, 4, weights="dirichlet")
    inp = workloads.fragment_inputs(cfg, list(range(len(sizes))), DEV)
    k, stride = inp.theta_L.shape

    def buffers():
        b = dict(th=inp.theta_g.clone(), mo=inp.momentum.clone())
        if call == "rda":
            b["codes"], b["cb"], b["rng"] = dlc.outputs_for(k, stride, len(sizes), DEV)
            b["norms"] = torch.zeros((k, len(sizes)), dtype=torch.float64, device=DEV)
            need = dlc.dlc_rda_workspace_bytes(k, inp.tensors)
        else:
            b["accum"], b["codes"], b["cb"], b["rng"] = dlc.ring_buffers(inp.theta_L, len(sizes))
            need = dlc.dlc_ring_workspace_bytes(k, inp.tensors)
        b["ws"] = torch.empty(max(256, need), dtype=torch.uint8, device=DEV)
        # rows the call does not write (the ring writes one codebook and range row per
        # non-empty chunk) must compare equal between the eager and the graph buffers
        for key in ("codes", "cb", "rng"):
            b[key].zero_()
        return b

    def run(b):
        if call == "rda":
            dlc.dlc_rda_outer_step(b["th"], b["mo"], inp.theta_L, inp.tensors, inp.weights, b["codes"], b["cb"],
                                   b["rng"], b["norms"], b["ws"])
        else:
            dlc.dlc_ring_outer_step(b["th"], b["mo"], inp.theta_L, inp.tensors, b["accum"], b["codes"], b["cb"],
                                    b["rng"], b["ws"])

    eager = buffers()
    run(eager)
    torch.cuda.synchronize()
    b = buffers()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            run(b)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    keys = ["th", "mo", "cb", "rng"] + (["norms"] if call == "rda" else [])
    for rep in range(3):
        b["th"].copy_(inp.theta_g)
        b["mo"].copy_(inp.momentum)
        noise = torch.randn(1 << 20, device=DEV).sum()  # unrelated eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.isfinite(noise)
        for key in keys:
            assert torch.equal(b[key], eager[key]), (rep, key)
