"""Outer-step merge throughput on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload c3|c4|c1|c2|c5k1|c5k16]

A step is one pass of the whole hot path over one batch of synthetic input:
pseudo-gradient statistics (dlc_quantize_range), clip + bucketize + histogram +
encode + codebook (dlc_quantize_encode), and dequantize + weighted mean + Nesterov
(dlc_merge_outer_step), over every tensor of the workload's call.  Inputs are
resident in HBM before timing starts.  Prints ONE JSON line.

Algorithmic bytes per merged parameter with K present learners:
  stats 4 + 4K (read), encode 4 + 4K (read) + K (codes written), merge K + 8 (read)
  + 8 (write)  ->  24 + 10K in total.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0
# the kernels and the block partition that launches them: both shape the HBM traffic
KERNEL_SOURCES = [os.path.join(ROOT, "diloco_outer_step_amd", "csrc", f) for f in ("dlc_kernels.hip", "dlc_api.hip")]
TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "traffic.json")


def kernel_source_hash():
    """SHA-256 (first 16 hex digits) of the kernel and launch sources with their
    comments and blank lines removed: a change to the code invalidates the counter
    record, a change to a comment does not."""
    h = hashlib.sha256()
    for path in KERNEL_SOURCES:
        with open(path, encoding="utf-8") as f:
            for line in f:
                code = line.split("//", 1)[0].rstrip()
                if code:
                    h.update(code.encode() + b"\n")
    return h.hexdigest()[:16]


def measured_traffic(kernel, workload):
    """HBM bytes per launch from the committed counter record, or None when the
    kernel source changed since the counters were taken."""
    try:
        rec = json.load(open(TRAFFIC_RECORD))
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    entry = rec.get("kernels", {}).get(workload, {}).get(kernel)
    return None if entry is None else entry.get("hbm_gb_per_launch")
METRIC = "outer-step merge params/s and HBM GB/s (% of peak) at K learners, 1 GPU"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="c3", choices=["c1", "c2", "c3", "c4", "c5k1", "c5k16"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true", help="skip the 10B-fragment line")
    ap.add_argument("--reported", action="store_true",
                    help="time the reported, ungated sets (4096^2 cold, the 10B set's largest fragment, "
                         "24-fragment cycles of the 135M set and of the edge mix, the next rows' calls) "
                         "and print them as one JSON line")
    ap.add_argument("--reported-only", default=None,
                    help="comma-separated subset of c1,c4_largest,c2,c5k1,c5k16,native_c2,native_c5k1,"
                         "broadcast_c3,stale_c3,ring_study,ring_c3,rda_c3")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a device-to-device copy of known size (counter calibration)")
    return ap.parse_args()


def fragment_ids(cfg, which):
    """Tensor ids of the median (or largest) fragment of the P-fragment plan."""
    import diloco_outer_step_amd as dlc
    numel = [s.numel for s in cfg.tensors]
    frag, loads = dlc.dlc_fragment_plan(numel, cfg.n_fragments)
    order = sorted(range(cfg.n_fragments), key=lambda p: (loads[p], p))
    p = order[cfg.n_fragments // 2] if which == "median" else order[-1]
    return [t for t, f in enumerate(frag) if f == p], p


def build_workload(key, device, which="median"):
    import workloads
    cfg = workloads.config(key)
    if cfg.n_fragments == 1:
        ids, frag = list(range(len(cfg.tensors))), 0
        desc = f"{cfg.title}; one outer step over all {len(ids)} tensors"
    else:
        ids, frag = fragment_ids(cfg, which)
        desc = f"{cfg.title}; {which} fragment {frag} of {cfg.n_fragments} ({len(ids)} tensors)"
    inp = workloads.fragment_inputs(cfg, ids, device, fragment=frag)
    return cfg, inp, desc


class Runner:
    """Buffers and the three stage calls of one outer step."""

    def __init__(self, inp, lr, beta):
        import diloco_outer_step_amd as dlc
        self.dlc = dlc
        self.inp = inp
        k, stride = inp.theta_L.shape
        self.codes, self.cb, self.rng = dlc.outputs_for(k, stride, len(inp.tensors), inp.theta_L.device)
        self.ws = dlc.alloc_workspace(k, inp.tensors, inp.theta_L.device)
        self.theta = inp.theta_g.clone()
        self.mom = inp.momentum.clone()
        self.lr, self.beta = lr, beta

    def stage_range(self):
        self.dlc.dlc_quantize_range(self.theta, self.inp.theta_L, self.inp.tensors, self.rng, self.ws,
                                    present=self.inp.present)

    def stage_encode(self):
        self.dlc.dlc_quantize_encode(self.theta, self.inp.theta_L, self.inp.tensors, self.rng, self.codes,
                                     self.cb, self.ws, present=self.inp.present)

    def stage_merge(self):
        self.dlc.dlc_merge_outer_step(self.theta, self.mom, self.codes, self.cb, self.inp.weights,
                                      self.inp.tensors, self.lr, self.beta)


def time_workload(key, steps, warmup, device, which="median"):
    import torch
    cfg, inp, desc = build_workload(key, device, which)
    torch.cuda.synchronize()
    n_params = sum(n for _, _, n in inp.tensors)
    kp = sum(1 for p in inp.present if p)
    r = Runner(inp, cfg.lr, cfg.beta)
    stages = [("stats", r.stage_range), ("encode", r.stage_encode), ("merge", r.stage_merge)]
    for _ in range(warmup):
        for _, fn in stages:
            fn()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)] for _ in range(steps)]
    t0 = time.perf_counter()
    for s in range(steps):
        ev[s][0].record(stream)
        for j, (_, fn) in enumerate(stages):
            fn()
            ev[s][j + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    stage_ms = {name: sum(ev[s][j].elapsed_time(ev[s][j + 1]) for s in range(steps)) / steps
                for j, (name, _) in enumerate(stages)}
    step_ms = sum(ev[s][0].elapsed_time(ev[s][-1]) for s in range(steps)) / steps
    per_param = {"stats": 4 + 4 * kp, "encode": 4 + 5 * kp, "merge": 16 + kp}
    total_bytes = (24 + 10 * kp) * n_params
    out = dict(workload=key, desc=desc, n_params=n_params, n_tensors=len(inp.tensors), k_present=kp,
               step_ms=step_ms, wall_ms_per_step=wall * 1e3 / steps, stage_ms=stage_ms,
               params_per_s=n_params / (step_ms * 1e-3),
               hbm_gbps=total_bytes / (step_ms * 1e-3) / 1e9,
               stage_gbps={k: per_param[k] * n_params / (stage_ms[k] * 1e-3) / 1e9 for k in stage_ms},
               bytes_per_param=24 + 10 * kp, stage_bytes_per_param=per_param, inp=inp, cfg=cfg)
    del r
    return out


class FragmentCall:
    """The three calls of one fragment's outer step on shared theta, momentum and
    codes buffers (per-fragment range, codebook and workspace)."""

    def __init__(self, inp, sel, theta, mom, codes, lr, beta):
        import diloco_outer_step_amd as dlc
        self.dlc = dlc
        self.inp, self.theta, self.mom, self.codes = inp, theta, mom, codes
        self.tensors = [inp.tensors[t] for t in sel]
        k = inp.theta_L.shape[0]
        _, self.cb, self.rng = dlc.outputs_for(k, 64, len(self.tensors), inp.theta_L.device)
        self.ws = dlc.alloc_workspace(k, self.tensors, inp.theta_L.device)
        self.lr, self.beta = lr, beta
        self.n_params = sum(n for _, _, n in self.tensors)
        self.k_present = sum(1 for p in inp.present if p)

    def __call__(self):
        d, inp = self.dlc, self.inp
        d.dlc_quantize_range(self.theta, inp.theta_L, self.tensors, self.rng, self.ws, present=inp.present)
        d.dlc_quantize_encode(self.theta, inp.theta_L, self.tensors, self.rng, self.codes, self.cb, self.ws,
                              present=inp.present)
        d.dlc_merge_outer_step(self.theta, self.mom, self.codes, self.cb, inp.weights, self.tensors, self.lr,
                               self.beta)


def time_calls(calls, reps, warmup, before=None):
    """Median ms of each call over reps rounds, with events on the launch stream
    between consecutive calls; the calls of a round are enqueued back to back and
    synchronized once per round.  The optional `before` runs untimed ahead of
    every call (then each call is timed on its own)."""
    import statistics
    import torch
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        for c in calls:
            c()
    torch.cuda.synchronize()
    ms = [[] for _ in calls]
    rounds = []
    for _ in range(reps):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * len(calls))]
        for j, c in enumerate(calls):
            if before is not None:
                before()
            ev[2 * j].record(stream)
            c()
            ev[2 * j + 1].record(stream)
        torch.cuda.synchronize()
        for j in range(len(calls)):
            ms[j].append(ev[2 * j].elapsed_time(ev[2 * j + 1]))
        rounds.append(ev[0].elapsed_time(ev[-1]))
    return [statistics.median(m) for m in ms], statistics.median(rounds)


def fragment_cycle(key, device, reps=5, warmup=2):
    """Every fragment of the P-fragment plan merged in turn (one call each)."""
    import torch
    import diloco_outer_step_amd as dlc
    import workloads
    cfg = workloads.config(key)
    ids = list(range(len(cfg.tensors)))
    frag, _ = dlc.dlc_fragment_plan([s.numel for s in cfg.tensors], cfg.n_fragments)
    per, total_params, total_bytes = [], 0, 0
    if cfg.absent_p == 0.0:
        inp = workloads.fragment_inputs(cfg, ids, device)
        theta, mom = inp.theta_g.clone(), inp.momentum.clone()
        codes = torch.empty(inp.theta_L.shape, dtype=torch.uint8, device=device)
        calls = [FragmentCall(inp, [t for t in ids if frag[t] == p], theta, mom, codes, cfg.lr, cfg.beta)
                 for p in range(cfg.n_fragments) if any(f == p for f in frag)]
        ms, cycle_ms = time_calls(calls, reps, warmup)
        for c, m in zip(calls, ms):
            per.append(m)
            total_params += c.n_params
            total_bytes += (24 + 10 * c.k_present) * c.n_params
        del calls, inp, theta, mom, codes
    else:
        # learners absent per fragment: each fragment has its own replicas
        for p in range(cfg.n_fragments):
            sel = [t for t in ids if frag[t] == p]
            if not sel:
                continue
            inp = workloads.fragment_inputs(cfg, sel, device, fragment=p)
            theta, mom = inp.theta_g.clone(), inp.momentum.clone()
            codes = torch.empty(inp.theta_L.shape, dtype=torch.uint8, device=device)
            c = FragmentCall(inp, list(range(len(sel))), theta, mom, codes, cfg.lr, cfg.beta)
            per.append(time_calls([c], reps, warmup)[0][0])
            total_params += c.n_params
            total_bytes += (24 + 10 * c.k_present) * c.n_params
            del c, inp, theta, mom, codes
            torch.cuda.empty_cache()
    if cfg.absent_p != 0.0:
        cycle_ms = sum(per)  # fragments built one at a time: the sum of their medians
        timing = f"sum of per-fragment medians of {reps} (each fragment's replicas built in turn)"
    else:
        timing = f"three calls per fragment, enqueued back to back; median of {reps} cycles"
    return dict(workload=cfg.title, fragments=len(per), cycle_ms=cycle_ms, fragment_ms=per, timing=timing,
                params=total_params, params_per_s=total_params / (cycle_ms * 1e-3),
                hbm_gbps=total_bytes / (cycle_ms * 1e-3) / 1e9,
                hbm_frac=total_bytes / (cycle_ms * 1e-3) / 1e9 / PEAK_HBM_GBPS)


def single_call_cold(key, device, reps=20, warmup=3, scratch_bytes=512 << 20):
    """One call over the whole set, median of reps, each after a scratch write
    large enough to evict the caches (256 MB Infinity Cache)."""
    import torch
    import workloads
    cfg = workloads.config(key)
    ids = list(range(len(cfg.tensors)))
    inp = workloads.fragment_inputs(cfg, ids, device)
    theta, mom = inp.theta_g.clone(), inp.momentum.clone()
    codes = torch.empty(inp.theta_L.shape, dtype=torch.uint8, device=device)
    c = FragmentCall(inp, ids, theta, mom, codes, cfg.lr, cfg.beta)
    scratch = torch.empty(scratch_bytes // 4, dtype=torch.float32, device=device)
    ms = time_calls([c], reps, warmup, before=lambda: scratch.fill_(1.0))[0][0]
    b = (24 + 10 * c.k_present) * c.n_params
    return dict(workload=cfg.title, ms=ms, params=c.n_params, params_per_s=c.n_params / (ms * 1e-3),
                hbm_gbps=b / (ms * 1e-3) / 1e9, hbm_frac=b / (ms * 1e-3) / 1e9 / PEAK_HBM_GBPS,
                cold_cache=f"{scratch_bytes >> 20} MB scratch write before each call")


def native_cycle(key, device, reps=5, warmup=2):
    """The whole fragment cycle through dlc_outer_cycle: quantize and merge on one
    stream, on two overlapped streams, on two streams with the update sent back to
    the learners (dlc_broadcast after each merge), with consecutive fragments on
    alternating lanes (DLC_TWO_LANES), on three and four lanes (dlc_outer_cycle_lanes),
    and the three- and four-lane cycles captured in a HIP graph and replayed; then the
    cycle merged by Radial-Directional Averaging (dlc_outer_cycle_rda) on one and four
    lanes and from a graph.  Four lanes match the four hardware queues a process gets
    here; more lanes share them and measured slower."""
    import statistics
    import torch
    import diloco_outer_step_amd as dlc
    import workloads
    cfg = workloads.config(key)
    ids = list(range(len(cfg.tensors)))
    inp = workloads.fragment_inputs(cfg, ids, device)
    frag, _ = dlc.dlc_fragment_plan([s.numel for s in cfg.tensors], cfg.n_fragments)
    grouped, first, _ = dlc.group_by_fragment(inp.tensors, frag, cfg.n_fragments)
    k, stride = inp.theta_L.shape
    weights = [list(inp.weights)] * cfg.n_fragments
    codes, cb, rng = dlc.outputs_for(k, stride, len(grouped), device)
    ws = torch.empty(max(256, 4 * (dlc.dlc_cycle_workspace_bytes(k, grouped, first) + 256)), dtype=torch.uint8,
                     device=device)
    theta, mom, theta_L = inp.theta_g.clone(), inp.momentum.clone(), inp.theta_L.clone()
    qs = torch.cuda.current_stream()
    ms = torch.cuda.Stream()
    n_params = sum(n for _, _, n in grouped)
    out = {}
    lane_streams = [qs, ms, torch.cuda.Stream(), torch.cuda.Stream()]
    for name, merge_stream, bc, lanes in (("one_stream", qs, False, False), ("two_streams", ms, False, False),
                                          ("two_streams_send_back", ms, True, False),
                                          ("two_lanes", ms, False, True), ("three_lanes", ms, False, 3),
                                          ("four_lanes", ms, False, 4)):
        def run():
            if lanes in (3, 4):
                dlc.dlc_outer_cycle_lanes(theta, mom, inp.theta_L, grouped, first, weights, codes, cb, rng, ws,
                                          lane_streams[:lanes])
                return
            dlc.dlc_outer_cycle(theta, mom, theta_L if bc else inp.theta_L, grouped, first, weights, codes, cb, rng,
                                ws, broadcast=bc, quantize_stream=qs, merge_stream=merge_stream, two_lanes=lanes)
        for _ in range(warmup):
            run()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(qs)
            run()
            e1.record(qs)  # the quantize stream joins the merge stream at the end of a cycle
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        ms_ = statistics.median(ts)
        b = (24 + 10 * k + (4 + 4 * k if bc else 0)) * n_params
        out[name] = dict(cycle_ms=ms_, params_per_s=n_params / (ms_ * 1e-3), hbm_gbps=b / (ms_ * 1e-3) / 1e9,
                         bytes_per_param=b // n_params)
    # the three- and four-lane cycles captured once in a HIP graph and replayed: no
    # host launch cost
    for n_lanes in (3, 4):
        graph, side = torch.cuda.CUDAGraph(), torch.cuda.Stream()
        others = [torch.cuda.Stream() for _ in range(n_lanes - 1)]
        side.wait_stream(qs)
        with torch.cuda.stream(side):
            with torch.cuda.graph(graph, stream=side):
                dlc.dlc_outer_cycle_lanes(theta, mom, inp.theta_L, grouped, first, weights, codes, cb, rng, ws,
                                          [side] + others)
        qs.wait_stream(side)
        for _ in range(warmup):
            graph.replay()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(qs)
            graph.replay()
            e1.record(qs)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        ms_ = statistics.median(ts)
        b = (24 + 10 * k) * n_params
        out[("three" if n_lanes == 3 else "four") + "_lanes_graph"] = dict(
            cycle_ms=ms_, params_per_s=n_params / (ms_ * 1e-3), hbm_gbps=b / (ms_ * 1e-3) / 1e9,
            bytes_per_param=b // n_params)
        del graph

    def timed(run):
        for _ in range(warmup):
            run()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(qs)
            run()
            e1.record(qs)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        return statistics.median(ts)

    # every fragment merged by Radial-Directional Averaging (dlc_outer_cycle_rda;
    # 24 + 11K bytes per parameter: one more read of the codes for the direction
    # norm): one lane, four lanes, and four lanes replayed from a HIP graph
    norms = torch.zeros((k, len(grouped)), dtype=torch.float64, device=device)
    ws_rda = torch.empty(4 * (dlc.dlc_cycle_rda_workspace_bytes(k, grouped, first) + 256), dtype=torch.uint8,
                         device=device)
    b = (24 + 11 * k) * n_params

    def rda(streams):
        dlc.dlc_outer_cycle_rda(theta, mom, inp.theta_L, grouped, first, weights, codes, cb, rng, norms, ws_rda,
                                streams)

    def entry(ms_):
        return dict(cycle_ms=ms_, params_per_s=n_params / (ms_ * 1e-3), hbm_gbps=b / (ms_ * 1e-3) / 1e9,
                    bytes_per_param=b // n_params)

    out["rda_one_lane"] = entry(timed(lambda: rda(lane_streams[:1])))
    out["rda_four_lanes"] = entry(timed(lambda: rda(lane_streams)))
    graph, side = torch.cuda.CUDAGraph(), torch.cuda.Stream()
    others = [torch.cuda.Stream() for _ in range(3)]
    side.wait_stream(qs)
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            rda([side] + others)
    qs.wait_stream(side)
    out["rda_four_lanes_graph"] = entry(timed(graph.replay))
    del graph
    out["workload"] = cfg.title
    out["fragments"] = cfg.n_fragments
    return out


def broadcast_rate(key, device, reps=5, warmup=2):
    """dlc_broadcast over every tensor of a set: 4 + 4K bytes per parameter."""
    import statistics
    import torch
    import diloco_outer_step_amd as dlc
    import workloads
    cfg = workloads.config(key)
    inp = workloads.fragment_inputs(cfg, list(range(len(cfg.tensors))), device)
    k = inp.theta_L.shape[0]
    theta_L = inp.theta_L
    for _ in range(warmup):
        dlc.dlc_broadcast(inp.theta_g, theta_L, inp.tensors)
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        dlc.dlc_broadcast(inp.theta_g, theta_L, inp.tensors)
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    ms_ = statistics.median(ts)
    n = sum(x for _, _, x in inp.tensors)
    b = (4 + 4 * k) * n
    return dict(workload=cfg.title, ms=ms_, params=n, learners=k, hbm_gbps=b / (ms_ * 1e-3) / 1e9,
                hbm_frac=b / (ms_ * 1e-3) / 1e9 / PEAK_HBM_GBPS)


def stale_rate(key, device, reps=5, warmup=2):
    """dlc_quantize_bases with the learners split between two bases (even learners
    against theta_g, odd ones against an older copy): one pass per base, so the
    statistics and encode passes read 4 + 4K bytes per parameter more than once
    only for the second base (2 * 4 + 4K each)."""
    import statistics
    import torch
    import diloco_outer_step_amd as dlc
    import workloads
    cfg = workloads.config(key)
    inp = workloads.fragment_inputs(cfg, list(range(len(cfg.tensors))), device)
    k, stride = inp.theta_L.shape
    old = inp.theta_g.clone()
    bases = [inp.theta_g if i % 2 == 0 else old for i in range(k)]
    codes, cb, rng = dlc.outputs_for(k, stride, len(inp.tensors), device)
    ws = dlc.alloc_workspace(k, inp.tensors, device)
    for _ in range(warmup):
        dlc.dlc_quantize_bases(bases, inp.theta_L, inp.tensors, codes, cb, rng, ws)
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        dlc.dlc_quantize_bases(bases, inp.theta_L, inp.tensors, codes, cb, rng, ws)
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    ms_ = statistics.median(ts)
    n = sum(x for _, _, x in inp.tensors)
    b = (2 * 4 + 4 * k + 2 * 4 + 5 * k) * n
    return dict(workload=cfg.title, bases=2, ms=ms_, params=n, learners=k, hbm_gbps=b / (ms_ * 1e-3) / 1e9,
                hbm_frac=b / (ms_ * 1e-3) / 1e9 / PEAK_HBM_GBPS)


def ring_study(device, ks=(2, 4, 8, 14, 16, 32, 64), n_params=1 << 24):
    """The ring with requantization at every hop against the star merge: relative
    RMS error of the merged pseudo-gradient against the exact fp64 mean, for
    growing K (4 tensors of n_params / 4, Delta ~ N(0, (1e-3)^2), theta ~ N(0,
    0.02^2)); g is read back from the Nesterov step from zero momentum,
    theta' = theta - lr (1 + beta) g."""
    import torch
    import diloco_outer_step_amd as dlc
    lr, beta = 0.7, 0.9
    q = n_params // 4
    tensors = [(i * q, i * q, q) for i in range(4)]
    g = torch.Generator(device=device)
    g.manual_seed(123)
    theta = torch.randn(n_params, generator=g, device=device) * 0.02
    out = []
    for k in ks:
        theta_L = torch.stack([theta - torch.randn(n_params, generator=g, device=device) * 1e-3 for _ in range(k)])
        exact = (theta.double()[None, :] - theta_L.double()).mean(0)
        mom = torch.zeros_like(theta)
        res = {}
        # star: each pseudo-gradient quantized once, equal weights
        codes, cb, rng = dlc.outputs_for(k, n_params, 4, device)
        ws = dlc.alloc_workspace(k, tensors, device)
        th, mo = theta.clone(), mom.clone()
        dlc.dlc_quantize(theta, theta_L, tensors, codes, cb, rng, ws)
        dlc.dlc_merge_outer_step(th, mo, codes, cb, [1.0] * k, tensors, lr, beta)
        res["star"] = th
        del codes, cb, rng, ws
        accum, codes, cb, rng = dlc.ring_buffers(theta_L, 4)
        ws = torch.empty(max(256, dlc.dlc_ring_workspace_bytes(k, tensors)), dtype=torch.uint8, device=device)
        th, mo = theta.clone(), mom.clone()
        dlc.dlc_ring_outer_step(th, mo, theta_L, tensors, accum, codes, cb, rng, ws, lr, beta)
        res["ring"] = th
        torch.cuda.synchronize()
        ref = float(exact.pow(2).mean().sqrt())
        row = {"k": k}
        for name, th in res.items():
            gk = (theta.double() - th.double()) / (lr * (1 + beta))
            row[name + "_rel_rms_error"] = float((gk - exact).pow(2).mean().sqrt()) / ref
        row["ring_over_star"] = row["ring_rel_rms_error"] / row["star_rel_rms_error"]
        out.append(row)
        del theta_L, accum, codes, cb, rng, ws, res
        torch.cuda.empty_cache()
    return out


def ring_rate(key, device, reps=3, warmup=1):
    """dlc_ring_outer_step over every tensor of a set, beside the star step."""
    import statistics
    import torch
    import diloco_outer_step_amd as dlc
    import workloads
    cfg = workloads.config(key)
    inp = workloads.fragment_inputs(cfg, list(range(len(cfg.tensors))), device)
    k = inp.theta_L.shape[0]
    accum, codes, cb, rng = dlc.ring_buffers(inp.theta_L, len(inp.tensors))
    ws = torch.empty(max(256, dlc.dlc_ring_workspace_bytes(k, inp.tensors)), dtype=torch.uint8, device=device)
    th, mo = inp.theta_g.clone(), inp.momentum.clone()
    run = lambda: dlc.dlc_ring_outer_step(th, mo, inp.theta_L, inp.tensors, accum, codes, cb, rng, ws,
                                          cfg.lr, cfg.beta)
    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        run()
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    ms_ = statistics.median(ts)
    n = sum(x for _, _, x in inp.tensors)
    # hop 0 quantizes the pseudo-gradients (stats 8, encode 9); every add reads
    # theta_g, theta_L and a code, writes the sum and forms the next message's
    # statistics (13); later hops and the gather only encode (5); merge 17 (one
    # learner): 18K + 16 for K >= 2
    b = (17 + 13 * (k - 1) + 5 * (k - 1) + 17) * n if k >= 2 else 34 * n
    return dict(workload=cfg.title, ms=ms_, params=n, learners=k, params_per_s=n / (ms_ * 1e-3),
                hbm_gbps=b / (ms_ * 1e-3) / 1e9, bytes_per_param=b // n)


def rda_rate(key, device, reps=5, warmup=2):
    """dlc_rda_outer_step over every tensor of a set."""
    import statistics
    import torch
    import diloco_outer_step_amd as dlc
    import workloads
    cfg = workloads.config(key)
    inp = workloads.fragment_inputs(cfg, list(range(len(cfg.tensors))), device)
    k, stride = inp.theta_L.shape
    t = len(inp.tensors)
    codes, cb, rng = dlc.outputs_for(k, stride, t, device)
    norms = torch.zeros((k, t), dtype=torch.float64, device=device)
    ws = torch.empty(max(256, dlc.dlc_rda_workspace_bytes(k, inp.tensors)), dtype=torch.uint8, device=device)
    th, mo = inp.theta_g.clone(), inp.momentum.clone()
    run = lambda: dlc.dlc_rda_outer_step(th, mo, inp.theta_L, inp.tensors, inp.weights, codes, cb, rng, norms, ws,
                                         cfg.lr, cfg.beta)
    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        run()
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    ms_ = statistics.median(ts)
    n = sum(x for _, _, x in inp.tensors)
    kp = sum(1 for w in inp.weights if w > 0)
    b = (24 + 11 * kp) * n  # the star step's 24 + 10K plus one more read of the codes
    return dict(workload=cfg.title, ms=ms_, params=n, learners=kp, params_per_s=n / (ms_ * 1e-3),
                hbm_gbps=b / (ms_ * 1e-3) / 1e9, hbm_frac=b / (ms_ * 1e-3) / 8e12, bytes_per_param=24 + 11 * kp)


def reported(device, only=None):
    """The parameter sets that are reported but not gated: the 4096^2 tensor (cold
    cache), the 10B set's largest fragment, full 24-fragment cycles of the 135M set
    and of the edge mix, and the calls of the next rows on the 1B set."""
    import torch
    keys = only.split(",") if only else ["c1", "c4_largest", "c2", "c5k1", "c5k16", "native_c2", "native_c5k1",
                                         "broadcast_c3",
                                         "stale_c3", "ring_study", "ring_c3", "rda_c3"]
    out = {}
    if "c1" in keys:
        out["c1"] = single_call_cold("c1", device)
        print(f"# c1 {out['c1']['ms']:.3f} ms", file=sys.stderr, flush=True)
    if "c4_largest" in keys:
        # the 10B set's largest fragment: one tensor of 525,336,576 params, K = 14
        res = time_workload("c4", 5, 2, device, which="largest")
        out["c4_largest"] = {k: res[k] for k in ("desc", "n_params", "n_tensors", "k_present", "step_ms",
                                                 "stage_ms", "params_per_s", "hbm_gbps", "stage_gbps",
                                                 "bytes_per_param")}
        out["c4_largest"]["hbm_frac"] = res["hbm_gbps"] / PEAK_HBM_GBPS
        del res
        torch.cuda.empty_cache()
        print(f"# c4 largest fragment {out['c4_largest']['step_ms']:.3f} ms, "
              f"{out['c4_largest']['hbm_gbps']:.0f} GB/s", file=sys.stderr, flush=True)
    for key in [k for k in keys if k.startswith("native_")]:
        out[key] = native_cycle(key[len("native_"):], device)
        torch.cuda.empty_cache()
        print(f"# {key}: " + ", ".join(f"{n} {v['cycle_ms']:.3f} ms" for n, v in out[key].items()
                                       if isinstance(v, dict)), file=sys.stderr, flush=True)
    if "rda_c3" in keys:
        out["rda_c3"] = rda_rate("c3", device)
        torch.cuda.empty_cache()
        print(f"# rda c3 {out['rda_c3']['ms']:.3f} ms", file=sys.stderr, flush=True)
    if "ring_study" in keys:
        out["ring_study"] = ring_study(device)
        torch.cuda.empty_cache()
        for row in out["ring_study"]:
            print(f"# ring study K={row['k']}: star {row['star_rel_rms_error']:.3e}, ring {row['ring_rel_rms_error']:.3e}",
                  file=sys.stderr, flush=True)
    if "ring_c3" in keys:
        out["ring_c3"] = ring_rate("c3", device)
        torch.cuda.empty_cache()
        print(f"# ring c3 {out['ring_c3']['ms']:.3f} ms", file=sys.stderr, flush=True)
    if "stale_c3" in keys:
        out["stale_c3"] = stale_rate("c3", device)
        torch.cuda.empty_cache()
        print(f"# stale quantize c3 {out['stale_c3']['ms']:.3f} ms", file=sys.stderr, flush=True)
    if "broadcast_c3" in keys:
        out["broadcast_c3"] = broadcast_rate("c3", device)
        torch.cuda.empty_cache()
        print(f"# broadcast c3 {out['broadcast_c3']['ms']:.3f} ms", file=sys.stderr, flush=True)
    for key in [k for k in keys if k in ("c2", "c5k1", "c5k16")]:
        out[key] = fragment_cycle(key, device)
        print(f"# {key} cycle {out[key]['cycle_ms']:.3f} ms over {out[key]['fragments']} fragments",
              file=sys.stderr, flush=True)
    return out


def copy_probe(device, nbytes=1 << 32, reps=5):
    import torch
    a = torch.empty(nbytes // 4, dtype=torch.float32, device=device)
    b = torch.empty_like(a)
    a.fill_(1.0)
    b.copy_(a)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    return dict(bytes_per_copy=2 * nbytes, ms=ms, gbps=2 * nbytes / (ms * 1e-3) / 1e9)


def cpu_baseline(res, budget_params=140_000_000):
    """Time the CPU oracle on a bounded sample of the same workload's tensors
    (host copies of exactly the inputs the GPU merged)."""
    import numpy as np
    import oracle
    inp = res["inp"]
    chosen, total = [], 0
    for t, (o, lo, n) in sorted(enumerate(inp.tensors), key=lambda x: -x[1][2]):
        if total + n > budget_params:
            continue
        chosen.append(t)
        total += n
    k = inp.theta_L.shape[0]
    stride = sum((inp.tensors[t][2] + 63) // 64 * 64 for t in chosen)
    th = np.zeros(stride, np.float32)
    mo = np.zeros(stride, np.float32)
    tl = np.zeros((k, stride), np.float32)
    sel, pos = [], 0
    for t in chosen:
        o, lo, n = inp.tensors[t]
        th[pos:pos + n] = inp.theta_g[o:o + n].cpu().numpy()
        mo[pos:pos + n] = inp.momentum[o:o + n].cpu().numpy()
        for i in range(k):
            if inp.present[i]:
                tl[i, pos:pos + n] = inp.theta_L[i, lo:lo + n].cpu().numpy()
        sel.append((pos, pos, n))
        pos += (n + 63) // 64 * 64
    t0 = time.perf_counter()
    oracle.outer_step(th, mo, tl, stride, sel, inp.weights, inp.present, res["cfg"].lr, res["cfg"].beta)
    dt = time.perf_counter() - t0
    out = dict(value=total / dt, unit="params/s", cores=1, kind="oracle",
               gbps=total * res["bytes_per_param"] / dt / 1e9,
               sample=f"{len(sel)} of the workload's tensors ({total} params, K={res['k_present']}) "
                      f"through oracle.outer_step (numpy, fp64, one thread); {dt:.1f} s",
               seconds=dt, numpy=np.__version__, cpu=cpu_model())
    try:
        out["parallel"] = cpu_baseline_parallel(res)
    except Exception as e:  # the single-process figure stands on its own
        out["parallel"] = {"error": f"{type(e).__name__}: {e}"}
    return out


# ---------------------------------------------------------------------------
# The oracle on a pool of host processes: (tensor, learner) quantization units,
# then one merge + Nesterov unit per tensor.  Workers are spawned (they never
# touch the GPU) and share the inputs through memory-mapped files.
_POOL = {}


def _pool_attach(spec):
    import numpy as np
    for name, (path, shape, dtype) in spec.items():
        _POOL[name] = np.memmap(path, dtype=dtype, mode="r+", shape=tuple(shape))


def _pool_quantize(unit):
    import oracle
    t, i, pos, n = unit
    x = oracle.pseudo_gradient(_POOL["th"][pos:pos + n], _POOL["tl"][i, pos:pos + n])
    q = oracle.quantize_tensor(x)
    _POOL["codes"][i, pos:pos + n] = q["codes"]
    _POOL["cb"][i, t] = q["codebook"]
    return 0


def _pool_merge(unit):
    import oracle
    t, pos, n, learners, w_hat, lr, beta = unit
    g = oracle.merge([_POOL["codes"][i, pos:pos + n] for i in learners], [_POOL["cb"][i, t] for i in learners],
                     [w_hat[i] for i in learners])
    th, mo = oracle.nesterov(_POOL["th"][pos:pos + n], _POOL["mo"][pos:pos + n], g, lr, beta)
    _POOL["th_out"][pos:pos + n] = th
    _POOL["mo_out"][pos:pos + n] = mo
    return 0


def pool_workers():
    """Worker processes for the oracle's pool: every core of this process's affinity
    mask, within the host's CPU share for this job where the environment states
    one (OMP_NUM_THREADS; 16 per GPU on the GPU hosts)."""
    cores = len(os.sched_getaffinity(0))
    share = os.environ.get("OMP_NUM_THREADS", "")
    return max(1, min(cores, int(share))) if share.isdigit() and int(share) > 0 else cores


def cpu_baseline_parallel(res, budget_params=48_000_000, max_workers=None, check=False):
    """The oracle's functions over a process pool, on host copies of mid-size
    tensors of the same workload (each at most a quarter of the sample, so the
    units balance).  check=True also returns the pool's theta and momentum with
    the sample's tensor list, for comparison with oracle.outer_step."""
    import multiprocessing as mp
    import tempfile
    import numpy as np
    import oracle
    inp = res["inp"]
    k = inp.theta_L.shape[0]
    learners = [i for i in range(k) if inp.present[i]]
    chosen, total = [], 0
    for t, (o, lo, n) in sorted(enumerate(inp.tensors), key=lambda x: -x[1][2]):
        if n > budget_params // 4 or total + n > budget_params:
            continue
        chosen.append(t)
        total += n
    if not chosen:
        return None
    stride = sum((inp.tensors[t][2] + 63) // 64 * 64 for t in chosen)
    workers = pool_workers() if max_workers is None else max(1, min(max_workers, pool_workers()))
    with tempfile.TemporaryDirectory() as tmp:
        spec = {"th": ([stride], "float32"), "mo": ([stride], "float32"), "tl": ([k, stride], "float32"),
                "codes": ([k, stride], "uint8"), "cb": ([k, len(chosen), 256], "float32"),
                "th_out": ([stride], "float32"), "mo_out": ([stride], "float32")}
        spec = {name: (os.path.join(tmp, name), shape, dt) for name, (shape, dt) in spec.items()}
        arr = {name: np.memmap(path, dtype=dt, mode="w+", shape=tuple(shape)) for name, (path, shape, dt) in spec.items()}
        units_q, units_m, pos = [], [], 0
        w_hat = oracle.normalize_weights(inp.weights)
        for j, t in enumerate(chosen):
            o, lo, n = inp.tensors[t]
            arr["th"][pos:pos + n] = inp.theta_g[o:o + n].cpu().numpy()
            arr["mo"][pos:pos + n] = inp.momentum[o:o + n].cpu().numpy()
            for i in learners:
                arr["tl"][i, pos:pos + n] = inp.theta_L[i, lo:lo + n].cpu().numpy()
                units_q.append((j, i, pos, n))
            units_m.append((j, pos, n, learners, w_hat, res["cfg"].lr, res["cfg"].beta))
            pos += (n + 63) // 64 * 64
        for a in arr.values():
            a.flush()
        ctx = mp.get_context("spawn")
        with ctx.Pool(workers, initializer=_pool_attach, initargs=(spec,)) as pool:
            pool.map(_pool_attach, [spec] * workers)  # workers up and attached before the clock starts
            t0 = time.perf_counter()
            units_q.sort(key=lambda u: -u[3])
            pool.map(_pool_quantize, units_q, chunksize=1)
            pool.map(_pool_merge, units_m, chunksize=1)
            dt = time.perf_counter() - t0
        if check:
            sel, pos = [], 0
            for t in chosen:
                sel.append((t, pos))
                pos += (inp.tensors[t][2] + 63) // 64 * 64
            return dict(theta=np.array(arr["th_out"]), momentum=np.array(arr["mo_out"]), tensors=sel)
    kp = len(learners)
    return dict(value=total / dt, unit="params/s", cores=workers, kind="oracle",
                gbps=total * (24 + 10 * kp) / dt / 1e9,
                sample=f"{len(chosen)} mid-size tensors of the workload ({total} params, K={kp}): "
                       f"oracle.quantize_tensor per (tensor, learner), then oracle.merge + oracle.nesterov "
                       f"per tensor, on a pool of {workers} spawned processes; {dt:.2f} s",
                seconds=dt, affinity_cores=len(os.sched_getaffinity(0)),
                omp_num_threads=os.environ.get("OMP_NUM_THREADS"))


def cpu_model():
    """The host CPU as /proc/cpuinfo names it: model name, family/model/stepping,
    physical cores and logical CPUs, and the cores this process may run on."""
    info = {}
    try:
        physical = set()
        phys_id = None
        for line in open("/proc/cpuinfo"):
            key, _, val = line.partition(":")
            key, val = key.strip(), val.strip()
            if key == "physical id":
                phys_id = val
            elif key == "core id":
                physical.add((phys_id, val))
            elif key in ("model name", "cpu family", "model", "stepping") and key not in info:
                info[key] = val
        if physical:
            info["physical_cores"] = len(physical)
    except OSError:
        info["model name"] = platform.processor()
    info["logical_cpus"] = os.cpu_count()
    info["affinity_cores"] = len(os.sched_getaffinity(0))
    return (f"{info.get('model name', '?')} (family {info.get('cpu family', '?')}, model {info.get('model', '?')}, "
            f"stepping {info.get('stepping', '?')}; {info.get('physical_cores', '?')} cores, "
            f"{info['logical_cpus']} logical CPUs, {info['affinity_cores']} in this process's affinity mask)")


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); "
              "the outer-step merge of one fragment runs on one device", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    device = "cuda:0"
    torch.cuda.set_device(0)
    if args.copy_probe:
        print(json.dumps({"copy_probe": copy_probe(device)}))
        return
    if args.reported:
        print(json.dumps({"reported": reported(device, args.reported_only)}), flush=True)
        return
    copy = copy_probe(device)
    print(f"# copy ceiling {copy['gbps']:.0f} GB/s", file=sys.stderr, flush=True)
    res = time_workload(args.workload, args.steps, args.warmup, device)
    print(f"# {res['workload']}: {res['step_ms']:.3f} ms/step, {res['hbm_gbps']:.0f} GB/s, "
          f"stages {res['stage_ms']}", file=sys.stderr, flush=True)
    dom = max(res["stage_ms"], key=res["stage_ms"].get)
    kernel_name = {"stats": "k_stats", "encode": "k_encode", "merge": "k_merge"}[dom]
    achieved = res["stage_gbps"][dom]
    algo_gb = res["stage_bytes_per_param"][dom] * res["n_params"] / 1e9
    line = {
        "metric": METRIC,
        "value": res["params_per_s"],
        "unit": "params/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": res["step_ms"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": res["desc"], "params_per_step": res["n_params"], "tensors": res["n_tensors"],
                   "learners_present": res["k_present"], "lr": res["cfg"].lr, "momentum": res["cfg"].beta,
                   "accumulation": "fp64 statistics and merge; bucket sums as fixed-point integers"},
        "hbm_gbps": res["hbm_gbps"],
        "hbm_frac": res["hbm_gbps"] / PEAK_HBM_GBPS,
        "bytes_per_param": res["bytes_per_param"],
        "stage_ms": res["stage_ms"],
        "stage_gbps": res["stage_gbps"],
        "roofline": {"bound": "hbm", "kernel": kernel_name, "achieved": achieved, "peak": PEAK_HBM_GBPS,
                     "unit": "GB/s", "frac": achieved / PEAK_HBM_GBPS,
                     "traffic": measured_traffic(kernel_name, args.workload),
                     "traffic_unit": "HBM GB per launch (counters)", "algorithmic_gb_per_launch": algo_gb,
                     "bytes_per_param": res["stage_bytes_per_param"][dom], "params_per_launch": res["n_params"],
                     "timing": f"HIP events around the {dom} stage on the launch stream"},
        "copy_ceiling_gbps": copy["gbps"],
    }
    # HBM bytes the counters saw per step (every kernel of the step, from the committed
    # record of the same kernel sources) over the measured step time; null otherwise
    counted = [measured_traffic(k, args.workload) for k in
               ("k_stats", "k_range", "k_encode", "k_hist_reduce", "k_codebook", "k_merge")]
    if all(c is not None for c in counted):
        line["counter_gbps"] = sum(counted) / (res["step_ms"] * 1e-3)
    else:
        line["counter_gbps"] = None
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(res)
        print(f"# cpu baseline {line['cpu_baseline']['value']:.3e} params/s", file=sys.stderr, flush=True)
    del res["inp"]
    torch.cuda.empty_cache()
    if args.workload == "c3" and not args.no_secondary:
        sec = time_workload("c4", max(3, args.steps // 2), 2, device)
        line["secondary"] = {"workload": sec["desc"], "params_per_s": sec["params_per_s"],
                             "ms_per_step": sec["step_ms"], "hbm_gbps": sec["hbm_gbps"],
                             "hbm_frac": sec["hbm_gbps"] / PEAK_HBM_GBPS, "stage_ms": sec["stage_ms"],
                             "stage_gbps": sec["stage_gbps"], "learners_present": sec["k_present"]}
        print(f"# c4: {sec['step_ms']:.3f} ms/step, {sec['hbm_gbps']:.0f} GB/s", file=sys.stderr, flush=True)
        del sec
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
