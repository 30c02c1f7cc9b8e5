#!/usr/bin/env python3
"""Benchmark of the selective-scan hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step is one full selective scan (every kernel of selscan_fwd /
selscan_mamba2_fwd) over one batch of seeded synthetic inputs that are
resident in HBM before the timed region starts.  Inputs and outputs rotate
over several copies when a workload is smaller than 1 GB, so the 256 MB
Infinity Cache cannot serve a step from the previous step's data.

Prints ONE JSON line: throughput in state updates per second
(batch * L * channels * d_state per step), the achieved HBM bandwidth of the
algorithmic bytes against the MI355X peak, the other workloads' figures, and
the fp64 CPU oracle timed on this host's cores.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E peak, GB/s
VALU_PEAK_LANE_OPS = 256 * 64 * 2.4e9   # 256 CUs x 64 fp32 lanes/clk x 2.4 GHz (non-packed)
HEADLINE = "mamba130m_l2k"
EXTRA = ["mamba2p8b_l8k", "long_1m", "mamba2_mh"]


def parse():
    p = argparse.ArgumentParser(description=__doc__.splitlines()[1])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default=HEADLINE)
    p.add_argument("--extra", default=",".join(EXTRA),
                   help="comma-separated extra workloads timed in the same run ('' for none)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--profile", action="store_true",
                   help="only warm up and run the timed steps of --workload (for rocprofv3)")
    p.add_argument("--seed", type=int, default=0)
    return p.parse_args()


def _call(ss, w, inp, out):
    if w.kind == "m1":
        return ss.fwd(inp["u"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"], inp["z"], inp["delta_bias"],
                      softplus=True, out=out[0], last_state=out[1])
    return ss.mamba2_fwd(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"], inp["z"], inp["dt_bias"],
                         softplus=True, out=out[0], last_state=out[1])


def time_workload(name, steps, warmup, seed, device):
    import torch
    import selective_state_space_25_amd as ss
    import synth

    w = synth.WORKLOADS[name]
    nbytes = synth.algorithmic_bytes(w)
    copies = 1 if nbytes >= (1 << 30) else max(2, int((1 << 30) // max(nbytes, 1)) + 1)
    copies = min(copies, 8)
    inps, outs = [], []
    for c in range(copies):
        inp = synth.workload_inputs(w, seed=seed + c, device=device)
        inps.append(inp)
        if w.kind == "m1":
            y = torch.empty((w.batch, w.dim, w.seqlen), dtype=w.out_dtype, device=device)
            last = torch.empty((w.batch, w.dim, w.dstate), dtype=torch.float32, device=device)
        else:
            y = torch.empty((w.batch, w.seqlen, w.nheads, w.headdim), dtype=w.out_dtype, device=device)
            last = torch.empty((w.batch, w.nheads, w.headdim, w.dstate), dtype=torch.float32, device=device)
        outs.append((y, last))
    stream = torch.cuda.current_stream(device)
    for i in range(warmup):
        _call(ss, w, inps[i % copies], outs[i % copies])
    torch.cuda.synchronize(device)
    # per-call events on the stream the kernels run on
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    t0 = time.perf_counter()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for i in range(steps):
        ev[i][0].record(stream)
        _call(ss, w, inps[i % copies], outs[i % copies])
        ev[i][1].record(stream)
    end.record(stream)
    torch.cuda.synchronize(device)
    wall = time.perf_counter() - t0
    total_ms = start.elapsed_time(end)
    per_call = sorted(a.elapsed_time(b) for a, b in ev)
    avg_call = sum(per_call) / len(per_call)
    ms_per_step = total_ms / steps
    res = {
        "workload": name, "note": w.note, "dtype": str(w.dtype).replace("torch.", ""),
        "ms_per_step": ms_per_step, "avg_call_ms": avg_call, "median_call_ms": per_call[len(per_call) // 2],
        "min_call_ms": per_call[0], "wall_s": wall, "steps": steps, "rotating_copies": copies,
        "updates_per_step": w.updates, "algorithmic_bytes": nbytes,
        "state_updates_per_s": w.updates / (ms_per_step * 1e-3),
        "hbm_gbs": nbytes / (avg_call * 1e-3) / 1e9,
    }
    res["hbm_frac_of_peak"] = res["hbm_gbs"] / HBM_PEAK_GBS
    del inps, outs
    torch.cuda.empty_cache()
    return w, res


def cpu_baseline(name, seed, budget_s=12.0):
    """The fp64 oracle on this host's cores, on the same workload: whole
    (batch, channel) rows of the workload's inputs, as many as fit in the time
    budget (all of them for the small workloads)."""
    import numpy as np
    import torch
    import synth
    import oracle

    cores = len(os.sched_getaffinity(0))
    oracle.set_threads(cores)
    w = synth.WORKLOADS[name]
    if w.kind != "m1":
        raise ValueError("cpu baseline implemented for Mamba-1 workloads")
    # rows processed per batch element; grow until the budget is used
    inp = synth.m1_inputs(1, w.dim, w.dstate, w.seqlen, w.dtype, w.a_kind, seed=seed, device="cpu")
    rows_total = w.batch * w.dim
    done_rows, elapsed, calls = 0, 0.0, 0
    t_start = time.perf_counter()
    while done_rows < rows_total and elapsed < budget_s:
        t = time.perf_counter()
        oracle.m1(inp["u"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"], inp["z"], inp["delta_bias"])
        elapsed += time.perf_counter() - t
        done_rows += w.dim
        calls += 1
    _ = np, torch, t_start
    upd = done_rows * w.seqlen * w.dstate
    return {"value": upd / elapsed, "unit": "state-updates/s", "cores": cores, "kind": "oracle",
            "sample": f"{done_rows} of {rows_total} (batch, channel) rows of {name}, full L={w.seqlen}, "
                      f"N={w.dstate}, fp64, {calls} oracle call(s), {elapsed:.2f} s",
            "seconds": elapsed}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: --gpus {args.gpus} is not supported "
              "(this build has no multi-GPU path; every box here has one GPU)", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    device = torch.device("cuda:0")
    import selective_state_space_25_amd as ss
    ss.lib()  # fail loudly if the HIP library is missing

    w, head = time_workload(args.workload, args.steps, args.warmup, args.seed, device)
    if args.profile:
        print(json.dumps(head))
        return
    extras = {}
    for name in [e for e in args.extra.split(",") if e and e != args.workload]:
        _, r = time_workload(name, max(3, min(args.steps, 20)), 2, args.seed, device)
        extras[name] = r

    line = {
        "metric": "selective-scan state-updates/s (B*L*D*N)",
        "value": head["state_updates_per_s"],
        "unit": "state-updates/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 in, fp32 state and out" if w.dtype == torch.bfloat16 else "f32",
        "data": "synthetic (seeded; distributions of the workload definitions)",
        "config": {"workload": w.name, "batch": w.batch, "seqlen": w.seqlen, "dstate": w.dstate,
                   **({"dim": w.dim} if w.kind == "m1" else {"nheads": w.nheads, "headdim": w.headdim,
                                                             "ngroups": w.ngroups}),
                   "parallelism": "single GPU"},
        "hbm_gbs": head["hbm_gbs"],
        "hbm_frac_of_peak": head["hbm_frac_of_peak"],
        "roofline": {"bound": "hbm", "achieved": head["hbm_gbs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": head["hbm_frac_of_peak"], "traffic": None,
                     "kernel": "selscan_fwd (all kernels of one call)",
                     "avg_launch_ms": head["avg_call_ms"]},
        "workloads": {args.workload: head, **extras},
        "library": ss.version(),
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(args.workload, args.seed)
    print(json.dumps(line))


if __name__ == "__main__":
    main()
