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
# fp32 VALU lane-instructions per second: 256 CUs x 4 SIMDs x 64 lanes per 4 cycles x 2.4 GHz (an FMA is one;
# the 157.3 TFLOP/s vector figure counts an FMA as two flops and two packed lanes per instruction)
VALU_PEAK_LANE_OPS = 256 * 4 * 16 * 2.4e9
VALU_PEAK_LANE_OPS = 256 * 64 * 2.4e9   # 256 CUs x 64 fp32 lanes/clk x 2.4 GHz (non-packed)
# the largest single-GPU workload: the million-token Mamba-1 layer scan
HEADLINE = "long_1m"
EXTRA = ["mamba130m_l2k", "mamba2p8b_l8k", "mamba2p8b_l8k_alog", "long_1m_shard8", "mamba2_mh"]


def parse():
    p = argparse.ArgumentParser(description=__doc__.splitlines()[1])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default=HEADLINE)
    p.add_argument("--extra", default=",".join(EXTRA),
                   help="comma-separated extra workloads timed in the same run ('' for none)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--profile", action="store_true",
                   help="only warm up and run the timed steps of --workload (for rocprofv3)")
    p.add_argument("--seed", type=int, default=0)
    p.add_argument("--backward", action="store_true",
                   help="with --profile: time the gradients (selscan_bwd) of --workload instead")
    p.add_argument("--copy-gib", type=float, default=0.0,
                   help="with --profile: also run a plain copy of this many GiB and a half-line "
                        "strided read of the same size (known bytes, to calibrate HBM byte counters)")
    return p.parse_args()


def _call(ss, w, inp, out):
    if w.kind == "m1":
        return ss.fwd(inp["u"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"], inp["z"], inp["delta_bias"],
                      softplus=True, out=out[0], last_state=out[1], workspace=out[2])
    return ss.mamba2_fwd(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"], inp["z"], inp["dt_bias"],
                         softplus=True, out=out[0], last_state=out[1], workspace=out[2])


def _outputs(w, device):
    """y, last state and the library's workspace, allocated once (as a caller
    that runs the layer repeatedly would) rather than inside every call."""
    import torch
    import selective_state_space_25_amd as ss
    code = ss.BF16 if w.dtype == torch.bfloat16 else ss.F32
    ocode = ss.BF16 if w.out_dtype == torch.bfloat16 else ss.F32
    if w.kind == "m1":
        y = torch.empty((w.batch, w.dim, w.seqlen), dtype=w.out_dtype, device=device)
        last = torch.empty((w.batch, w.dim, w.dstate), dtype=torch.float32, device=device)
        nws = ss.workspace_bytes(w.batch, w.dim, w.dstate, w.seqlen, code, ocode)
    else:
        y = torch.empty((w.batch, w.seqlen, w.nheads, w.headdim), dtype=w.out_dtype, device=device)
        last = torch.empty((w.batch, w.nheads, w.headdim, w.dstate), dtype=torch.float32, device=device)
        nws = ss.mamba2_workspace_bytes(w.batch, w.seqlen, w.nheads, w.headdim, w.ngroups, w.dstate, code, ocode)
    ws = torch.empty(max(nws, 256), dtype=torch.uint8, device=device) if nws > 0 else None
    return y, last, ws


def _timed(ss, w, inps, outs, steps, stream):
    """Time `steps` calls back to back with events on the kernels' stream."""
    import torch
    copies = len(inps)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record(stream)
    for i in range(steps):
        ev[i][0].record(stream)
        _call(ss, w, inps[i % copies], outs[i % copies])
        ev[i][1].record(stream)
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return start.elapsed_time(end), sorted(a.elapsed_time(b) for a, b in ev), wall


def time_workload(name, steps, warmup, seed, device, kernel_timing=True, warm_s=0.0):
    """Region 1: `steps` plain calls (throughput).  Region 2: the same number
    of calls with every kernel bracketed by HIP events on the launch stream
    (per-kernel durations for the roofline of the dominant kernel).  Before
    them, `warmup` untimed calls, continued until `warm_s` seconds have passed
    (the clock needs ~0.1 s of load to settle: with 3 warm-up calls the
    Mamba-2 layer measured 0.19-0.21 ms per call, after 0.2 s of them 0.17)."""
    import torch
    import selective_state_space_25_amd as ss
    import synth

    w = synth.WORKLOADS[name]
    nbytes = synth.algorithmic_bytes(w)
    copies = 1 if nbytes >= (1 << 30) else max(2, int((1 << 30) // max(nbytes, 1)) + 1)
    copies = min(copies, 8)
    inps = [synth.workload_inputs(w, seed=seed + c, device=device) for c in range(copies)]
    outs = [_outputs(w, device) for _ in range(copies)]
    stream = torch.cuda.current_stream(device)
    t_warm = time.perf_counter()
    nwarm = 0
    while nwarm < warmup or time.perf_counter() - t_warm < warm_s:
        _call(ss, w, inps[nwarm % copies], outs[nwarm % copies])
        nwarm += 1
        if nwarm >= warmup and nwarm % 8 == 0:
            torch.cuda.synchronize(device)
    torch.cuda.synchronize(device)
    total_ms, per_call, wall = _timed(ss, w, inps, outs, steps, stream)
    avg_call = sum(per_call) / len(per_call)
    ms_per_step = total_ms / steps
    res = {
        "workload": name, "note": w.note, "dtype": str(w.dtype).replace("torch.", ""),
        "ms_per_step": ms_per_step, "avg_call_ms": avg_call, "median_call_ms": per_call[len(per_call) // 2],
        "min_call_ms": per_call[0], "wall_s": wall, "steps": steps, "warmup_calls": nwarm, "rotating_copies": copies,
        "updates_per_step": w.updates, "algorithmic_bytes": nbytes,
        "state_updates_per_s": w.updates / (ms_per_step * 1e-3),
        "hbm_gbs": nbytes / (ms_per_step * 1e-3) / 1e9,
    }
    res["hbm_frac_of_peak"] = res["hbm_gbs"] / HBM_PEAK_GBS
    if kernel_timing:
        ss.timing_collect()
        ss.timing_enable(True)
        try:
            _timed(ss, w, inps, outs, steps, stream)
        finally:
            ss.timing_enable(False)
        res["kernels"] = ss.timing_collect()
    del inps, outs
    torch.cuda.empty_cache()
    return w, res


def time_decode(name, steps, device):
    """One-token update (selscan_step / selscan_mamba2_step) at the batch and
    channel shape of a workload: HBM-bound on reading and writing the state."""
    import torch
    import selective_state_space_25_amd as ss
    import synth

    w = synth.WORKLOADS[name]
    if w.kind == "m1":
        inp = synth.m1_inputs(w.batch, w.dim, w.dstate, 1, w.dtype, w.a_kind, seed=0, device=device)
        state = torch.zeros((w.batch, w.dim, w.dstate), dtype=torch.float32, device=device)
        args = [inp[k][..., 0].contiguous() if inp[k] is not None and inp[k].dim() == 3 else inp[k]
                for k in ("u", "delta", "A", "B", "C", "D", "z", "delta_bias")]
        f = lambda: ss.step(state, *args)
        bound, _ = ss.bind_step(state, *args)
        es = torch.tensor([], dtype=w.dtype).element_size()
        rows = w.batch * w.dim
        nbytes = rows * w.dstate * 4 * 2 + rows * (3 * es + 4) + 2 * w.batch * w.dstate * es + w.dim * (w.dstate + 2) * 4
    else:
        inp = synth.m2_inputs(w.batch, 1, w.nheads, w.headdim, w.ngroups, w.dstate, w.dtype, seed=0, device=device)
        state = torch.zeros((w.batch, w.nheads, w.headdim, w.dstate), dtype=torch.float32, device=device)
        args = [inp[k][:, 0].contiguous() if inp[k] is not None and inp[k].dim() >= 3 else inp[k]
                for k in ("x", "dt", "A", "B", "C", "D", "z", "dt_bias")]
        f = lambda: ss.mamba2_step(state, *args)
        bound, _ = ss.bind_mamba2_step(state, *args)
        es = torch.tensor([], dtype=w.dtype).element_size()
        rows = w.batch * w.nheads * w.headdim
        nbytes = (rows * w.dstate * 4 * 2 + rows * (2 * es + 4) + w.batch * w.nheads * es
                  + 2 * w.batch * w.ngroups * w.dstate * es + 3 * w.nheads * 4)
    for _ in range(5):
        f()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    stream = torch.cuda.current_stream(device)
    e0.record(stream)
    for _ in range(steps):
        f()
    e1.record(stream)
    torch.cuda.synchronize()
    us_call = e0.elapsed_time(e1) * 1e3 / steps
    # the same steps through a call bound once (arguments marshalled at
    # binding), and the host time of the C-ABI call alone (wall clock per
    # call, kernels left to run behind it)
    for _ in range(5):
        bound()
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(steps):
        bound()
    e1.record(stream)
    torch.cuda.synchronize()
    us_bound = e0.elapsed_time(e1) * 1e3 / steps
    t = time.perf_counter()
    for _ in range(steps):
        bound()
    us_host = (time.perf_counter() - t) * 1e6 / steps
    torch.cuda.synchronize()
    # The kernels alone: the call above is bound by the host issuing it, and
    # events around one small launch add their own microseconds, so the
    # steps are captured once as a graph of back-to-back launches (kernel
    # nodes only) and the replay is timed.
    how = "graph of back-to-back launches"
    try:
        side = torch.cuda.Stream(device)
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            for _ in range(3):
                f()
        stream.wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(steps):
                f()
        g.replay()
        torch.cuda.synchronize()
        e0.record(stream)
        g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / steps
        del g
    except RuntimeError:
        how = "events around each launch"
        ss.timing_collect()
        ss.timing_enable(True)
        try:
            for _ in range(steps):
                f()
            torch.cuda.synchronize()
        finally:
            ss.timing_enable(False)
        us = list(ss.timing_collect().values())[0]["avg_ms"] * 1e3
    return {"shape_of": name, "us_per_token_kernel": us, "kernel_timing": how,
            "us_per_token_call": us_call, "us_per_token_bound_call": us_bound,
            "host_us_per_bound_call": us_host, "bytes_per_token": nbytes, "kernel_gbs": nbytes / (us * 1e-6) / 1e9,
            "kernel_state_updates_per_s": rows * w.dstate / (us * 1e-6)}


def time_conv1d(name, steps, device, width=4):
    """Causal depthwise conv (+ SiLU) over a workload's u-shaped input, bf16
    in and out: an HBM stream (one read of x, one write of out)."""
    import torch
    import selective_state_space_25_amd as ss
    import synth

    w = synth.WORKLOADS[name]
    g = torch.Generator(device=device).manual_seed(0)
    x = torch.randn((w.batch, w.dim, w.seqlen), generator=g, device=device, dtype=torch.float32).to(w.dtype)
    wt = torch.randn((w.dim, width), generator=g, device=device, dtype=torch.float32) * 0.5
    bias = torch.randn((w.dim,), generator=g, device=device, dtype=torch.float32)
    out = torch.empty_like(x)
    f = lambda: ss.conv1d(x, wt, bias, silu=True, out=out)
    for _ in range(3):
        f()
    torch.cuda.synchronize()
    ss.timing_collect()
    ss.timing_enable(True)
    try:
        for _ in range(steps):
            f()
        torch.cuda.synchronize()
    finally:
        ss.timing_enable(False)
    k = list(ss.timing_collect().values())[0]
    nbytes = 2 * x.numel() * x.element_size() + (w.dim * (width + 1)) * 4
    return {"shape_of": name, "width": width, "dtype": str(w.dtype).replace("torch.", ""),
            "kernel_ms": k["avg_ms"], "bytes": nbytes, "gbs": nbytes / (k["avg_ms"] * 1e-3) / 1e9,
            "frac_of_hbm_peak": nbytes / (k["avg_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS}


def time_backward(name, steps, device, warmup=2, seed=0):
    """Gradients (selscan_bwd / selscan_mamba2_bwd: every input's gradient
    from dout) on a workload's full shape, fp32 dout and gradients, workspace
    preallocated."""
    import torch
    import selective_state_space_25_amd as ss
    import synth

    w = synth.WORKLOADS[name]
    inp = synth.workload_inputs(w, seed=seed, device=device)
    code = ss.BF16 if w.dtype == torch.bfloat16 else ss.F32
    if w.kind == "m1":
        dout = synth.m1_dout(w.batch, w.dim, w.seqlen, torch.float32, seed=seed, device=device)
        ws = torch.empty(ss.bwd_workspace_bytes(w.batch, w.dim, w.dstate, w.seqlen, code, ss.F32),
                         dtype=torch.uint8, device=device)
        f = lambda: ss.bwd(inp["u"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"], inp["z"],
                           inp["delta_bias"], dout, softplus=True, workspace=ws)
    else:
        dout = synth.m2_dout(w.batch, w.seqlen, w.nheads, w.headdim, torch.float32, seed=seed, device=device)
        ws = torch.empty(ss.mamba2_bwd_workspace_bytes(w.batch, w.seqlen, w.nheads, w.headdim, w.ngroups, w.dstate,
                                                       code, ss.F32), dtype=torch.uint8, device=device)
        f = lambda: ss.mamba2_bwd(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"], inp["z"],
                                  inp["dt_bias"], dout, softplus=True, workspace=ws)
    for _ in range(warmup):
        f()
    torch.cuda.synchronize(device)
    stream = torch.cuda.current_stream(device)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(steps):
        f()
    end.record(stream)
    torch.cuda.synchronize(device)
    ms = start.elapsed_time(end) / steps
    ss.timing_collect()
    ss.timing_enable(True)
    try:
        for _ in range(steps):
            f()
        torch.cuda.synchronize(device)
    finally:
        ss.timing_enable(False)
    kernels = ss.timing_collect()
    nbytes = synth.bwd_algorithmic_bytes(w)
    res = {"shape_of": name, "ms_per_call": ms, "steps": steps, "dout_dtype": "float32", "grad_dtype": "float32",
           "state_updates_per_s": w.updates / (ms * 1e-3), "algorithmic_bytes": nbytes,
           "hbm_gbs": nbytes / (ms * 1e-3) / 1e9, "hbm_frac_of_peak": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
           "kernels": kernels}
    del inp, dout, ws
    torch.cuda.empty_cache()
    return res


def time_abi_host(calls=200):
    """Host time per decode call through the C ABI alone: the native harness
    built beside the library (abi_bench) calls the step entry points back to
    back from C++.  None when it is not built."""
    import subprocess
    exe = os.path.join(os.path.dirname(os.path.abspath(__file__)), "selective_state_space_25_amd", "abi_bench")
    if not os.path.exists(exe):
        return None
    r = subprocess.run([exe, str(calls)], capture_output=True, text=True, timeout=120)
    if r.returncode != 0:
        return {"error": r.stderr.strip()[-300:]}
    return json.loads(r.stdout.strip().splitlines()[-1])


def copy_calibration(device, gib):
    """Kernels of known traffic for scaling the HBM byte counters: a plain copy
    (torch.neg over fp32, reads and writes `gib` GiB) and a read of the first
    64 bytes of every 128-byte line of a `gib` GiB bf16 buffer."""
    import torch
    n = int(gib * (1 << 30)) // 4
    src = torch.ones(n, dtype=torch.float32, device=device)
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.neg(src, out=dst)
    del src, dst
    xb = torch.ones(n * 4 // 128, 64, dtype=torch.bfloat16, device=device)
    for _ in range(3):
        half = xb[:, :32].contiguous()
    del xb, half
    torch.cuda.synchronize(device)
    return n * 4


def time_copy(device, gib=1.0, reps=10):
    """Achievable HBM bandwidth for context: a plain device copy of `gib` GiB
    (fp32, read once and written once), timed with events on the current
    stream; GB/s counts the bytes read plus the bytes written."""
    import torch
    n = int(gib * (1 << 30)) // 4
    src = torch.ones(n, dtype=torch.float32, device=device)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    st = torch.cuda.current_stream(device)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize(device)
    e0.record(st)
    for _ in range(reps):
        dst.copy_(src)
    e1.record(st)
    torch.cuda.synchronize(device)
    ms = e0.elapsed_time(e1) / reps
    del src, dst
    return {"bytes": 2 * n * 4, "ms": ms, "gbs": 2 * n * 4 / (ms * 1e-3) / 1e9}


def decay_path(w):
    """Which Mamba-1 decay path the workload's A takes: "structured" when every
    row has A[d, n] == fl32((n + 1) A[d, 0]) (one exponential per token),
    else "general" (one per state update)."""
    if w.kind != "m1":
        return "scalar per head"
    import torch
    import synth
    A = synth.a_matrix(w.dim, w.dstate, w.a_kind, 0)
    n1 = torch.arange(1, w.dstate + 1, dtype=torch.float32)
    s = (A == n1[None, :] * A[:, :1]).all(dim=1)
    return "structured" if bool(s.all()) else ("general" if not bool(s.any()) else "mixed")


def dominant_kernel(res):
    name, k = max(res["kernels"].items(), key=lambda kv: kv[1]["total_ms"])
    return name, k


def read_profile(workload, kernel):
    """Fields of the committed rocprofv3 counter summary of `kernel` on
    `workload` (profiles/traffic_<kernel>_<workload>.txt), or {} when there
    is none or the kernel's source has changed since the counters were taken."""
    import hashlib
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles",
                        f"traffic_{kernel}_{workload}.txt")
    if not os.path.exists(path):
        return {}
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith(" "):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    src = kv.get("source")
    if not src or "source_sha256" not in kv:
        return {}
    spath = os.path.join(os.path.dirname(os.path.abspath(__file__)), src)
    if not os.path.exists(spath) or hashlib.sha256(open(spath, "rb").read()).hexdigest() != kv["source_sha256"]:
        return {}
    return kv


def read_traffic(workload, kernel):
    """HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, scaled) or None."""
    kv = read_profile(workload, kernel)
    return float(kv["hbm_bytes_per_launch"]) if "hbm_bytes_per_launch" in kv else None


def read_valu(workload, kernel, launch_ms=None, updates=None):
    """VALU lane-instructions per state update and VALU busy at the measured
    clock, from the same committed summary, or None.  With this run's launch
    time and the call's state updates, also the lane-instruction rate it
    implies against the VALU peak (the kernel's other roofline)."""
    kv = read_profile(workload, kernel)
    out = {}
    for k in ("valu_lane_ops_per_update", "valu_busy_at_measured_clock", "measured_clock_ghz"):
        if k in kv:
            out[k] = float(kv[k])
    if out and launch_ms and updates and "valu_lane_ops_per_update" in out:
        rate = out["valu_lane_ops_per_update"] * updates / (launch_ms * 1e-3)
        out.update({"achieved_lane_ops_per_s": rate, "peak_lane_ops_per_s": VALU_PEAK_LANE_OPS,
                    "frac": rate / VALU_PEAK_LANE_OPS})
    return out or None


def read_call_traffic(workload, kernel):
    """HBM bytes of the whole call (every kernel, counters scaled as for the
    dominant kernel) from the dominant kernel's committed summary, or None."""
    kv = read_profile(workload, kernel)
    if "call_hbm_bytes" not in kv:
        return None
    return {"bytes": float(kv["call_hbm_bytes"]), "over_algorithmic": float(kv["call_traffic_over_algorithmic"])}


def cpu_baseline(name, seed, min_s=10.0, max_s=30.0):
    """The fp64 oracle on this host's cores, on the same workload.  The
    whole workload is repeated until at least `min_s` seconds of oracle time
    have run; when one pass takes longer than `max_s`, a prefix of the
    (batch, channel) rows is used instead."""
    import numpy as np
    import synth
    import oracle

    cores = len(os.sched_getaffinity(0))
    env = os.environ.get("OMP_NUM_THREADS")
    if env and env.isdigit() and int(env) > 0:
        cores = min(cores, int(env))
    oracle.set_threads(cores)
    w = synth.WORKLOADS[name]
    if w.kind != "m1":
        raise ValueError("cpu baseline implemented for Mamba-1 workloads")
    elems = w.batch * w.dim * w.seqlen
    if elems <= (1 << 28):
        inp = synth.m1_inputs(w.batch, w.dim, w.dstate, w.seqlen, w.dtype, w.a_kind, seed=seed, device="cpu")
        what = f"{name}"
    else:
        # too large to hold in fp64 on the host: the first channels of batch
        # element 0 at the full length (the oracle's time is linear in rows)
        rows = max(1, (1 << 27) // w.seqlen)
        inp = synth.m1_row_sample(w, rows, seed=seed)
        what = f"the first {rows} of {w.dim} channels of batch element 0 of {name}"
    f64 = {k: (None if v is None else np.ascontiguousarray(v.double().numpy())) for k, v in inp.items()}
    nb, nd, nl = f64["u"].shape
    nn = f64["A"].shape[1]

    def one(rows_b):
        t = time.perf_counter()
        oracle.m1(f64["u"][:rows_b], f64["delta"][:rows_b], f64["A"], f64["B"][:rows_b], f64["C"][:rows_b],
                  f64["D"], f64["z"][:rows_b], f64["delta_bias"])
        return time.perf_counter() - t

    # probe with one batch element, then size the sample
    t1 = one(1)
    per_pass = t1 * nb
    rows_b = nb if per_pass <= max_s else max(1, int(max_s / t1))
    passes, elapsed = 0, 0.0
    while elapsed < min_s or passes == 0:
        elapsed += one(rows_b)
        passes += 1
    upd = passes * rows_b * nd * nl * nn
    res = {"value": upd / elapsed, "unit": "state-updates/s", "cores": cores, "kind": "oracle",
           "sample": f"{passes} pass(es) over {rows_b} of {nb} batch elements of {what} "
                     f"({rows_b * nd} (batch, channel) rows, full L={nl}, N={nn}), "
                     f"fp64 with {cores} OpenMP threads, {elapsed:.1f} s of oracle time",
           "seconds": elapsed, "per_core": upd / elapsed / cores, "cpu_model": cpu_model()}
    res["one_core"] = one_core_baseline(seed)
    oracle.set_threads(cores)
    return res


def cpu_model():
    """The host CPU's model name, from /proc/cpuinfo (None where absent)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def one_core_baseline(seed, min_s=2.0):
    """The oracle on one thread, for scaling context: one batch element of the
    Mamba-130m-shaped layer (1536 channels x 2048 tokens, N 16), repeated
    until `min_s` seconds have run."""
    import numpy as np
    import synth
    import oracle

    w = synth.WORKLOADS["mamba130m_l2k"]
    inp = synth.m1_inputs(1, w.dim, w.dstate, w.seqlen, w.dtype, w.a_kind, seed=seed, device="cpu")
    f64 = {k: (None if v is None else np.ascontiguousarray(v.double().numpy())) for k, v in inp.items()}
    oracle.set_threads(1)
    passes, elapsed = 0, 0.0
    while elapsed < min_s or passes == 0:
        t = time.perf_counter()
        oracle.m1(f64["u"], f64["delta"], f64["A"], f64["B"], f64["C"], f64["D"], f64["z"], f64["delta_bias"])
        elapsed += time.perf_counter() - t
        passes += 1
    upd = passes * w.dim * w.seqlen * w.dstate
    return {"value": upd / elapsed, "unit": "state-updates/s", "cores": 1,
            "sample": f"{passes} pass(es) over batch element 0 of mamba130m_l2k (1536 channels, L=2048, N=16)",
            "seconds": elapsed}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: --gpus {args.gpus} is not supported "
              "(the library has no multi-GPU path)", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    device = torch.device("cuda:0")
    import selective_state_space_25_amd as ss
    ss.lib()  # fail loudly if the HIP library is missing

    if args.profile and args.backward:
        res = time_backward(args.workload, args.steps, device, warmup=args.warmup, seed=args.seed)
        if args.copy_gib > 0:
            res["copy_calibration_bytes_each_way"] = copy_calibration(device, args.copy_gib)
        print(json.dumps(res))
        return
    w, head = time_workload(args.workload, args.steps, args.warmup, args.seed, device,
                            kernel_timing=not args.profile)
    if args.profile:
        if args.copy_gib > 0:
            head["copy_calibration_bytes_each_way"] = copy_calibration(device, args.copy_gib)
        print(json.dumps(head))
        return
    import synth
    extras = {}
    for name in [e for e in args.extra.split(",") if e and e != args.workload]:
        ew = synth.WORKLOADS[name]
        steps = max(10, min(args.steps, 50))
        _, r = time_workload(name, steps, 3, args.seed, device, warm_s=0.25)
        kn, kk = dominant_kernel(r)
        r["decay_path"] = decay_path(ew)
        r["dominant_kernel"] = {"name": kn, "avg_ms": kk["avg_ms"],
                                "gbs": r["algorithmic_bytes"] / (kk["avg_ms"] * 1e-3) / 1e9,
                                "frac": r["algorithmic_bytes"] / (kk["avg_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS,
                                "traffic": read_traffic(name, kn),
                                "valu": read_valu(name, kn, kk["avg_ms"], r["updates_per_step"]),
                                "call_traffic": read_call_traffic(name, kn)}
        extras[name] = r

    kname, k = dominant_kernel(head)
    avg_ms = k["avg_ms"]
    # the dominant (output) kernel reads every input once and writes y and
    # the final state: its algorithmic bytes per launch are the method's
    achieved = head["algorithmic_bytes"] / (avg_ms * 1e-3) / 1e9
    traffic = read_traffic(args.workload, kname)
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
        # the arithmetic of the path: every update, exponential and sum in fp32
        "dtype": "f32",
        "data": "synthetic (seeded; distributions of the workload definitions)",
        "config": {"workload": w.name, "batch": w.batch, "seqlen": w.seqlen, "dstate": w.dstate,
                   **({"dim": w.dim} if w.kind == "m1" else {"nheads": w.nheads, "headdim": w.headdim,
                                                             "ngroups": w.ngroups}),
                   "inputs": str(w.dtype).replace("torch.", ""), "state": "float32",
                   "output": str(w.out_dtype).replace("torch.", ""),
                   "decay_path": decay_path(w), "parallelism": "single GPU"},
        "hbm_gbs": head["hbm_gbs"],
        "hbm_frac_of_peak": head["hbm_frac_of_peak"],
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "kernel": kname, "avg_launch_ms": avg_ms, "launches": k["launches"],
                     "bytes_per_launch": head["algorithmic_bytes"],
                     "traffic_over_algorithmic": None if traffic is None else traffic / head["algorithmic_bytes"],
                     # the whole call (every kernel and the gaps between them)
                     "whole_call": {"achieved": head["hbm_gbs"], "frac": head["hbm_frac_of_peak"],
                                    "ms": head["ms_per_step"],
                                    "traffic": read_call_traffic(args.workload, kname)},
                     "kernels": {n: v["avg_ms"] for n, v in head["kernels"].items()},
                     # the same kernel against its other ceiling, the VALU issue rate
                     "valu": read_valu(args.workload, kname, avg_ms, head["updates_per_step"]),
                     "summary_pass": ({"traffic": read_traffic(args.workload, "m1_scan_summary"),
                                       "valu": read_valu(args.workload, "m1_scan_summary",
                                                         head["kernels"]["m1_scan_summary"]["avg_ms"],
                                                         head["updates_per_step"])}
                                      if "m1_scan_summary" in head["kernels"] else None)},
        "workloads": {args.workload: head, **extras},
        "library": ss.version(),
    }
    # the bandwidth a plain copy reaches on this GPU, next to the peak
    copy = time_copy(device)
    line["roofline"]["copy"] = {"gbs": copy["gbs"], "kernel_frac_of_copy": achieved / copy["gbs"],
                                "call_frac_of_copy": head["hbm_gbs"] / copy["gbs"]}
    line["decode"] = {n: time_decode(n, 200, device) for n in ("mamba2p8b_l8k", "mamba2_mh")}
    line["decode"]["c_abi_host_us_per_call"] = time_abi_host()
    line["conv1d"] = time_conv1d("mamba2p8b_l8k", 10, device)
    line["backward"] = {n: time_backward(n, 5 if n != "long_1m" else 3, device)
                        for n in ("mamba130m_l2k", "mamba2p8b_l8k", "long_1m", "mamba2_mh")}
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(args.workload, args.seed)
        line["cpu_baseline"]["gpu_over_cpu"] = line["value"] / line["cpu_baseline"]["value"]
    print(json.dumps(line))


if __name__ == "__main__":
    main()
