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
    h = hashlib.sha256()
    for path in KERNEL_SOURCES:
        with open(path, "rb") as f:
            h.update(f.read())
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


def build_workload(key, device):
    import workloads
    cfg = workloads.config(key)
    if cfg.n_fragments == 1:
        ids, frag = list(range(len(cfg.tensors))), 0
        desc = f"{cfg.title}; one outer step over all {len(ids)} tensors"
    else:
        ids, frag = fragment_ids(cfg, "median")
        desc = f"{cfg.title}; median fragment {frag} of {cfg.n_fragments} ({len(ids)} tensors)"
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


def time_workload(key, steps, warmup, device):
    import torch
    cfg, inp, desc = build_workload(key, device)
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


def cpu_baseline(res, budget_params=100_000_000):
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
    return dict(value=total / dt, unit="params/s", cores=1, kind="oracle",
                sample=f"{len(sel)} of the workload's tensors ({total} params, K={res['k_present']}) "
                       f"through oracle.outer_step (numpy, fp64, one thread); {dt:.1f} s",
                seconds=dt, numpy=np.__version__, cpu=cpu_model())


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor()


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
                   "accumulation": "fp64 statistics, histogram sums and merge"},
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
