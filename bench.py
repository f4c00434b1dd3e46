#!/usr/bin/env python3
"""Benchmark of the chunked gated delta rule forward on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic input
that is already resident in HBM: one gdn_chunk_fwd call (for bf16 inputs a
single kernel: gate cumsum, A, (I+A)^-1, the WY new values, state carry and
output), timed with HIP events on the stream it runs on.  fp32 workloads run
the two stage entry points and time each stage.  Other workloads: the decode
step (--workload decode_bf16), Gated DeltaNet-2 (--workload gdn2_bf16) and its
decode step (--workload decode2_bf16), and the backward of the chunked forward
on the layer-shaped inputs (--workload layer_bwd_bf16), the Gated DeltaNet-2
backward (--workload gdn2_bwd_bf16), and the whole layer
around the rule: prologue, chunked forward and gated RMSNorm
(--workload layer_full_bf16).

Default workload: B=8, H=8, T=4096, d_k=d_v=128, bf16 q/k/v, fp32 gates,
fp32 output and state (the layer-shaped case).  Prints ONE JSON line on
stdout; progress goes to stderr.

  python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "chunk_gated_delta_rule fwd tokens/s and % bf16 MFMA peak, T=4096 d=128"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_PEAK_TFLOPS = 2516.6      # MI355X dense bf16/fp16 MFMA, published
BT = 64


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# Sources each measured kernel is compiled from (besides build.py, whose flags
# shape every kernel): a traffic record stays valid while these are unchanged.
KERNEL_SOURCES = {
    "fused_kernel": ("gdn_fused.hip", "gdn_tile.h", "gdn_device.h"),
    "step_kernel": ("gdn_step.hip", "gdn_device.h"),
    "step2_kernel": ("gdn_step.hip", "gdn_device.h"),
    "gdn2_kernels": ("gdn2_fused.hip", "gdn_tile.h", "gdn_device.h"),
    "gdn_bwd": ("gdn_bwd.hip", "gdn_bwd_fused.hip", "gdn_fused.hip", "gdn_chunk.hip", "gdn_tile.h", "gdn_device.h"),
    "prologue_kernel": ("gdn_prologue.hip", "gdn_device.h"),
    "gdn2_bwd": ("gdn2_bwd.hip", "gdn2_chunk.hip", "gdn2_states.hip", "gdn_tile.h", "gdn_device.h"),
}


def source_sha(kernel: str = None) -> str:
    """Hash of the sources of `kernel` (all of csrc when None) and build.py."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "gated_delta_rule_34_amd", "csrc")
    if kernel is None:
        files = sorted(glob.glob(os.path.join(csrc, "*")))
    else:
        files = [os.path.join(csrc, f) for f in KERNEL_SOURCES[kernel]]
    files.append(os.path.join(ROOT, "gated_delta_rule_34_amd", "build.py"))
    for p in files:
        h.update(open(p, "rb").read())
    return h.hexdigest()[:16]


def read_traffic(kernel: str, workload: str):
    """HBM traffic per launch from a committed rocprofv3 --pmc summary, or None when
    no summary exists or the kernel sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("source_sha") != source_sha(kernel):
        return None
    try:
        return float(kv["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


SETTLE_S = 0.25   # default seconds of back-to-back steps before any timed region


def host_cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def percentile(xs, p):
    ys = sorted(xs)
    if not ys:
        return None
    k = (len(ys) - 1) * p / 100.0
    lo = int(k)
    hi = min(lo + 1, len(ys) - 1)
    return ys[lo] + (ys[hi] - ys[lo]) * (k - lo)


def run_timed(step, sets, args, per_launch_min: int = 50):
    """The timing protocol shared by every workload.

    1. `args.warmup` untimed steps, then more back-to-back steps until at least
       --settle-ms of load have run (the GPU clock needs ~50 ms of load to
       settle), whatever --warmup says.
    2. The timed region: exactly `args.steps` steps between two synchronisations,
       with one HIP event pair on the current stream around all of them (wall
       clock and event time).
    3. A distribution pass outside the timed region: max(steps, 50) steps, each
       between its own event pair, for the median / p10 / p90 of one step,
       followed at once by the library's clock probe, which reads the shader
       clock before the GPU idles.
    Returns a dict with ms_per_step (wall), event_ms_per_step and the stats."""
    import torch
    import gated_delta_rule_34_amd as gdn
    n = len(sets)
    t0 = time.perf_counter()
    done = 0
    for i in range(args.warmup):
        step(sets[i % n])
        done += 1
    torch.cuda.synchronize()
    while time.perf_counter() - t0 < args.settle_ms * 1e-3:
        for _ in range(20):
            step(sets[done % n])
            done += 1
        torch.cuda.synchronize()
    settle_s = time.perf_counter() - t0
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record()
    for i in range(args.steps):
        step(sets[i % n])
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    event_ms = e0.elapsed_time(e1) / args.steps
    m = max(args.steps, per_launch_min)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(m)]
    for i in range(m):
        evs[i][0].record()
        step(sets[i % n])
        evs[i][1].record()
    probe = gdn.clock_probe(nblocks=256, spin_us=2000)
    torch.cuda.synchronize()
    per = [a.elapsed_time(b) * 1e3 for a, b in evs]
    pc = probe.cpu().double()
    mhz = sorted((100.0 * pc[:, 0] / pc[:, 1]).tolist())
    shader_clock = {"median_mhz": mhz[len(mhz) // 2], "min_mhz": mhz[0], "max_mhz": mhz[-1], "workgroups": len(mhz),
                    "method": "s_memtime cycles over 100 MHz s_memrealtime ticks in a 2 ms probe kernel enqueued "
                              "right after the per-step launches (the clock just after the load, which can be "
                              "above the clock under it)"}
    return {"ms_per_step": wall * 1e3 / args.steps, "event_ms_per_step": event_ms,
            "settle": {"steps": done, "seconds": settle_s},
            "step_us": {"median": percentile(per, 50), "p10": percentile(per, 10), "p90": percentile(per, 90),
                        "n": m, "method": "one HIP event pair per step, outside the timed region"},
            "device_clock": shader_clock}


def timing_fields(tm):
    """JSON fields every workload reports from run_timed's result."""
    return {"settle": tm["settle"], "step_us": tm["step_us"], "device_clock": tm["device_clock"],
            "host_cpu": host_cpu_model()}


def to_dev(a, dev):
    import numpy as np
    import torch
    if a is None:
        return None
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def gdn_flops_full_tile(B, T, H, Dk, Dv):
    """Algorithmic MFMA flops of the chunked WY forward per the full-tile count:
    2*BT*(3*Dk + 2*Dv) + 6*Dk*Dv per token-head (A, W, U, intra output products
    and the three state products)."""
    return float(B) * T * H * (2 * BT * (3 * Dk + 2 * Dv) + 6 * Dk * Dv)


def walk_algorithmic_bytes(B, T, H, Dk, Dv, esz, h0):
    """Bytes the state walk must move by definition: q, k, v (input dtype), beta,
    o (fp32) once each, the final state (and h0) once.  The per-chunk intermediates
    of the intra stage are not counted."""
    per_tok = (2 * Dk + Dv) * esz + 4 + Dv * 4
    state = B * H * Dk * Dv * 4
    return float(B) * T * H * per_tok + state * (2 if h0 else 1)


def cpu_baseline_gdn(x):
    import oracle
    names = ("q", "k", "v", "g", "beta", "h0")
    args = [x[n + "_f64"] for n in names]
    B, T, H = x["B"], x["T"], x["H"]
    # sample: whole heads of the same workload, bounded to ~10-30 s of CPU work
    t0 = time.perf_counter()
    oracle.gdn_fwd(*[a[:1, :, :1] if a is not None else None for a in args[:5]], None)
    per_head = max(time.perf_counter() - t0, 1e-3)
    threads = oracle.max_threads()
    heads = B * H
    budget_heads = max(1, min(heads, int(20.0 * threads / per_head)))
    nb = max(1, min(B, budget_heads // H))
    sub = [a[:nb] if a is not None else None for a in args]
    t0 = time.perf_counter()
    oracle.gdn_fwd(*sub[:5], sub[5])
    dt = time.perf_counter() - t0
    # when the whole workload takes well under 10 s, repeat it up to ~10 s of work
    runs = max(1, min(40, int(10.0 / max(dt, 1e-3))))
    t0 = time.perf_counter()
    for _ in range(runs - 1):
        oracle.gdn_fwd(*sub[:5], sub[5])
    dt = (dt + time.perf_counter() - t0) / runs
    return {"value": nb * T / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{nb} of {B} sequences x {H} heads x {T} tokens (fp64 per-token recurrence, "
                      f"OpenMP over heads), {runs} run(s), {dt:.2f} s each"}


def bench_gdn(args, wl):
    import numpy as np
    import torch
    import gated_delta_rule_34_amd as gdn
    import gdn_inputs as gi

    dev = torch.device("cuda:0")
    t0 = time.perf_counter()
    x = gi.workload(wl)
    log(f"[bench] generated {wl} in {time.perf_counter() - t0:.1f}s")
    B, T, H, Dk, Dv = x["B"], x["T"], x["H"], x["Dk"], x["Dv"]
    NT = (T + BT - 1) // BT
    base = {n: to_dev(x[n], dev) for n in ("q", "k", "v", "g", "beta", "h0")}
    # Rotate independent buffer sets so the 256 MB Infinity Cache cannot serve
    # a step from the previous one.
    sets = []
    for i in range(args.sets):
        s = {n: (t.clone() if t is not None else None) for n, t in base.items()}
        s["o"] = torch.empty((B, T, H, Dv), dtype=torch.float32, device=dev)
        s["ht"] = torch.empty((B, H, Dk, Dv), dtype=torch.float32, device=dev)
        s["G2"] = torch.empty((B, H, NT, BT), dtype=torch.float32, device=dev)
        s["Tinv"] = torch.empty((B, H, NT, BT, BT), dtype=torch.float32, device=dev)
        sets.append(s)
    scale = x["scale"]
    fused = x["dtype"] == "bf16"   # bf16 inputs: one kernel; fp32: intra stage + walk
    ws = torch.empty(gdn.gdn_chunk_fwd_workspace(B, T, H, Dk, Dv, gdn.GDN_BF16 if fused else gdn.GDN_F32),
                     dtype=torch.uint8, device=dev)

    def step(s, ev=None):
        if ev is not None:
            ev[0].record()
        if fused:
            gdn.gdn_chunk_fwd(s["q"], s["k"], s["v"], s["g"], s["beta"], s["h0"], scale=scale, workspace=ws,
                              out=s["o"], final_state=s["ht"])
            if ev is not None:
                ev[1].record()
                ev[2].record()
            return
        gdn.gdn_chunk_intra(s["k"], s["g"], s["beta"], G2_out=s["G2"], Tinv_out=s["Tinv"])
        if ev is not None:
            ev[1].record()
        gdn.gdn_chunk_walk(s["q"], s["k"], s["v"], s["beta"], s["G2"], s["Tinv"], s["h0"], scale=scale,
                           out=s["o"], final_state=s["ht"])
        if ev is not None:
            ev[2].record()

    tm = run_timed(step, sets, args)
    ms = tm["ms_per_step"]
    # few heads and a long sequence: the library plans the chunk-parallel scan
    # (a workspace beyond 256 bytes), four launches per step
    scan = fused and ws.numel() > 256
    if scan:
        k1_ms, k2_ms = tm["event_ms_per_step"], 0.0
        kernels = {"chunk_parallel_step": k1_ms * 1e3}
    elif fused:
        # one kernel per step: the event pair around the timed region gives its
        # average launch duration without per-launch event gaps
        k1_ms, k2_ms = tm["event_ms_per_step"], 0.0
        kernels = {"fused_kernel": k1_ms * 1e3}
    else:
        # the two stages, each between events, in a pass of its own after the timed region
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
        for i in range(args.steps):
            step(sets[i % len(sets)], evs[i])
        torch.cuda.synchronize()
        k1_ms = sum(e[0].elapsed_time(e[1]) for e in evs) / args.steps
        k2_ms = sum(e[1].elapsed_time(e[2]) for e in evs) / args.steps
        kernels = {"intra_kernel": k1_ms * 1e3, "walk_kernel": k2_ms * 1e3}
    log(f"[bench] {args.steps} steps: {ms:.4f} ms/step wall; per launch (HIP events): " +
        ", ".join(f"{k} {v:.1f} us" for k, v in kernels.items()) +
        f"; step median {tm['step_us']['median']:.1f} us (p10 {tm['step_us']['p10']:.1f}, "
        f"p90 {tm['step_us']['p90']:.1f}); clock {tm['device_clock']}")

    tokens = B * T
    flops = gdn_flops_full_tile(B, T, H, Dk, Dv)
    esz = 2 if x["dtype"] == "bf16" else 4
    has_h0 = x["h0"] is not None
    if scan:
        # the whole step: output-free segment walks, the scan, the single kernel
        # on the segments and the final-state copy
        kname, kms = "fused_walk_kernel+seg_scan_kernel+fused_kernel+seg_final_kernel", k1_ms
        kbytes = walk_algorithmic_bytes(B, T, H, Dk, Dv, esz, has_h0) + 4.0 * B * T * H
    elif fused:
        kname, kms = "fused_kernel", k1_ms
        kbytes = walk_algorithmic_bytes(B, T, H, Dk, Dv, esz, has_h0) + 4.0 * B * T * H   # + g
    elif k2_ms >= k1_ms:
        kname, kms = "walk_kernel", k2_ms
        kbytes = walk_algorithmic_bytes(B, T, H, Dk, Dv, esz, has_h0)
    else:
        kname, kms = "intra_kernel", k1_ms
        kbytes = float(B) * T * H * (Dk * esz + 8 + 4) + B * H * NT * BT * BT * 4.0
    achieved = kbytes / (kms * 1e-3) / 1e9
    traffic = read_traffic(kname, wl)
    res = {
        "metric": METRIC,
        "value": tokens / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if x["dtype"] == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": wl, "B": B, "T": T, "H": H, "Dk": Dk, "Dv": Dv, "chunk": BT,
                   "inputs": x["dtype"], "state_and_output": "fp32",
                   "mfma": ("bf16 operands (inputs, state hi + lo parts) and fp16 operands (T - I, P, new "
                            "values), fp32 accumulate") if x["dtype"] == "bf16" else "fp32",
                   "h0": has_h0, "buffer_sets": args.sets, "parallelism": "single GPU",
                   "kernels": ("chunk-parallel state scan (segment walks, scan, single kernel on the segments)"
                               if scan else "single fused kernel" if fused else "intra-chunk stage + state walk")},
        "roofline": {"bound": "hbm", "kernel": kname, "achieved": achieved, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "algorithmic_bytes_per_launch": kbytes, "avg_launch_us": kms * 1e3,
                     "traffic": traffic},
        "mfma": {"algorithmic_tflops": flops / (ms * 1e-3) / 1e12, "peak_tflops": MFMA_PEAK_TFLOPS,
                 "frac": flops / (ms * 1e-3) / 1e12 / MFMA_PEAK_TFLOPS,
                 "flop_model": "full-tile 2*64*(3*Dk+2*Dv)+6*Dk*Dv per token-head"},
        "kernels_us": kernels,
        **timing_fields(tm),
    }
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle baseline")
        res["cpu_baseline"] = cpu_baseline_gdn(x)
    else:
        res["cpu_baseline"] = None
    return res


def bench_gdn2(args, wl):
    import torch
    import gated_delta_rule_34_amd as gdn
    import gdn_inputs as gi
    import oracle

    dev = torch.device("cuda:0")
    x = gi.workload(wl)
    B, T, H, Dk, Dv = x["B"], x["T"], x["H"], x["Dk"], x["Dv"]
    names = ("q", "k", "v", "log_alpha", "b", "w", "h0")
    base = {n: to_dev(x[n], dev) for n in names}
    sets = []
    for i in range(args.sets):
        s = {n: (t.clone() if t is not None else None) for n, t in base.items()}
        s["o"] = torch.empty((B, T, H, Dv), dtype=torch.float32, device=dev)
        s["ht"] = torch.empty((B, H, Dk, Dv), dtype=torch.float32, device=dev)
        sets.append(s)
    code = gdn.GDN_BF16 if x["dtype"] == "bf16" else gdn.GDN_F32
    ws = torch.empty(gdn.gdn2_chunk_fwd_workspace(B, T, H, Dk, Dv, code), dtype=torch.uint8, device=dev)

    def step(s):
        gdn.gdn2_chunk_fwd(*[s[n] for n in names], scale=x["scale"], workspace=ws, out=s["o"],
                           final_state=s["ht"])

    tm = run_timed(step, sets, args)
    ms = tm["ms_per_step"]
    kms = tm["event_ms_per_step"]
    esz = 2 if x["dtype"] == "bf16" else 4
    # q, k, b (Dk) and v, w (Dv) in the input dtype, log_alpha fp32, o fp32, final state
    kbytes = float(B) * T * H * ((3 * Dk + 2 * Dv) * esz + 4 * Dk + 4 * Dv) + B * H * Dk * Dv * 4.0
    achieved = kbytes / (kms * 1e-3) / 1e9
    flops = gdn_flops_full_tile(B, T, H, Dk, Dv)
    # bf16 inputs take the fused prep + walk pair, fp32 inputs the staged pair
    kname = ("gdn2_prep_kernel+gdn2_pipe_kernel+gdn2_walk_fused_kernel" if esz == 2 else "gdn2_intra_kernel+gdn2_walk_kernel")
    res = {
        "metric": "chunk gated delta rule-2 fwd tokens/s, T=4096 d=128",
        "value": B * T / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16" if esz == 2 else "f32", "data": "synthetic",
        "config": {"workload": wl, "B": B, "T": T, "H": H, "Dk": Dk, "Dv": Dv, "chunk": BT,
                   "inputs": x["dtype"], "kernels": "gdn2 intra-chunk stage + state walk",
                   "buffer_sets": args.sets, "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "kernel": kname, "achieved": achieved,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "algorithmic_bytes_per_launch": kbytes, "avg_launch_us": kms * 1e3,
                     "traffic": read_traffic("gdn2_kernels", wl) if esz == 2 else None},
        "mfma": {"algorithmic_tflops": flops / (ms * 1e-3) / 1e12, "peak_tflops": MFMA_PEAK_TFLOPS,
                 "frac": flops / (ms * 1e-3) / 1e12 / MFMA_PEAK_TFLOPS,
                 "flop_model": "full-tile 2*64*(3*Dk+2*Dv)+6*Dk*Dv per token-head"},
        **timing_fields(tm),
    }
    if not args.no_cpu_baseline:
        args64 = [x[n + "_f64"] for n in names]
        # one sequence's heads, repeated for about 10 s of work
        nb = 1
        sub = [a[:nb] if a is not None else None for a in args64[:6]]
        t0 = time.perf_counter()
        runs = 0
        while runs == 0 or (time.perf_counter() - t0 < 10.0 and runs < 200):
            oracle.gdn2_fwd(*sub, None)
            runs += 1
        dt = (time.perf_counter() - t0) / runs
        res["cpu_baseline"] = {"value": nb * T / dt, "unit": "tokens/s", "cores": oracle.max_threads(),
                               "kind": "oracle",
                               "sample": f"{nb} of {B} sequences x {H} heads x {T} tokens, {runs} run(s), "
                                         f"{dt:.2f} s each"}
    else:
        res["cpu_baseline"] = None
    return res


# The two decode steps: input names, entry point, oracle, kernel, extra bytes per head.
STEPS = {
    "decode_bf16": dict(names=("q", "k", "v", "g", "beta"), fn="gdn_recurrent_step", ref="gdn_step",
                        kernel="step_kernel", label="gdn_recurrent_step", gate_bytes=lambda Dk, Dv, es: 8),
    "decode2_bf16": dict(names=("q", "k", "v", "log_alpha", "b", "w"), fn="gdn2_recurrent_step", ref="gdn2_step",
                         kernel="step2_kernel", label="gdn2_recurrent_step",
                         gate_bytes=lambda Dk, Dv, es: 4 * Dk + es * (Dk + Dv)),
}


def bench_step(args, wl):
    import torch
    import gated_delta_rule_34_amd as gdn
    import gdn_inputs as gi
    import oracle

    spec = STEPS[wl]
    dev = torch.device("cuda:0")
    x = gi.workload(wl)
    B, H, Dk, Dv = x["B"], x["H"], x["Dk"], x["Dv"]
    names = spec["names"]
    base = {n: to_dev(x[n], dev) for n in names + ("S",)}
    sets = []
    for i in range(args.sets):
        s = {n: t.clone() for n, t in base.items()}
        s["o"] = torch.empty((B, H, Dv), dtype=torch.float32, device=dev)
        sets.append(s)
    fn = getattr(gdn, spec["fn"])

    def step(s):
        fn(*[s[n] for n in names], s["S"], scale=x["scale"], out=s["o"])

    tm = run_timed(step, sets, args)
    ms = tm["ms_per_step"]
    kms = tm["event_ms_per_step"]
    esz = 2 if x["dtype"] == "bf16" else 4
    # state read and written once, q, k, v, the gates, and o
    kbytes = float(B) * H * (2 * Dk * Dv * 4 + (2 * Dk + Dv) * esz + spec["gate_bytes"](Dk, Dv, esz) + Dv * 4)
    achieved = kbytes / (kms * 1e-3) / 1e9
    res = {
        "metric": f"{spec['label']} decode tokens/s (HBM roofline), B={B} H={H} d={Dk}",
        "value": B / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": wl, "B": B, "H": H, "Dk": Dk, "Dv": Dv, "inputs": x["dtype"],
                   "state": "fp32 in place", "buffer_sets": args.sets, "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "kernel": spec["kernel"], "achieved": achieved, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS, "algorithmic_bytes_per_launch": kbytes,
                     "avg_launch_us": kms * 1e3, "traffic": read_traffic(spec["kernel"], wl)},
        **timing_fields(tm),
    }
    if not args.no_cpu_baseline:
        args_f64 = [x[n + "_f64"] for n in names + ("S",)]
        ref = getattr(oracle, spec["ref"])
        t0 = time.perf_counter()
        reps = 0
        while time.perf_counter() - t0 < 10.0:
            ref(*args_f64)
            reps += 1
        dt = (time.perf_counter() - t0) / reps
        res["cpu_baseline"] = {"value": B / dt, "unit": "tokens/s", "cores": oracle.max_threads(),
                               "kind": "oracle", "sample": f"whole decode batch, {reps} repetitions in ~10 s"}
    else:
        res["cpu_baseline"] = None
    return res


# The two backwards: input names, entry point, oracle, extra gate bytes per token-head.
BWDS = {
    "layer_bwd_bf16": dict(names=("q", "k", "v", "g", "beta"), fn="gdn_chunk_bwd", ws="gdn_chunk_bwd_workspace",
                           ref="gdn_bwd", kernel="gdn_bwd", label="chunk_gated_delta_rule bwd",
                           extra=lambda Dk, Dv, es: 8 + 8),             # g, beta in; dg, dbeta out
    "gdn2_bwd_bf16": dict(names=("q", "k", "v", "log_alpha", "b", "w"), fn="gdn2_chunk_bwd",
                          ws="gdn2_chunk_bwd_workspace", ref="gdn2_bwd", kernel="gdn2_bwd",
                          label="chunk gated delta rule-2 bwd",
                          # b, w and log_alpha in; dlog_alpha, db, dw out
                          extra=lambda Dk, Dv, es: (Dk + Dv) * es + 4 * Dk + (2 * Dk + Dv) * 4),
}


def bench_bwd(args, wl):
    """Backward of a chunked forward on its workload's inputs: one step = every
    backward stage over the whole batch."""
    import numpy as np
    import torch
    import gated_delta_rule_34_amd as gdn
    import gdn_inputs as gi

    spec = BWDS[wl]
    dev = torch.device("cuda:0")
    x = gi.workload(wl)
    B, T, H, Dk, Dv = x["B"], x["T"], x["H"], x["Dk"], x["Dv"]
    rng = np.random.default_rng(x.get("seed", 0) + 7)
    do = rng.standard_normal((B, T, H, Dv)).astype(np.float32)
    dht = rng.standard_normal((B, H, Dk, Dv)).astype(np.float32)
    names = spec["names"]
    base = {n: to_dev(x[n], dev) for n in names}
    base["do"] = to_dev(do, dev)
    base["dht"] = to_dev(dht, dev)
    sets = [{n: t.clone() for n, t in base.items()} for _ in range(args.sets)]
    dt = gdn.GDN_BF16 if x["dtype"] == "bf16" else gdn.GDN_F32
    ws = torch.empty(getattr(gdn, spec["ws"])(B, T, H, Dk, Dv, dt), dtype=torch.uint8, device=dev)
    fn = getattr(gdn, spec["fn"])

    def step(s):
        fn(*[s[n] for n in names], None, s["do"], s["dht"], scale=x["scale"], workspace=ws)

    tm = run_timed(step, sets, args)
    ms = tm["ms_per_step"]
    kms = tm["event_ms_per_step"]
    esz = 2 if x["dtype"] == "bf16" else 4
    # inputs q, k, v (and the gates), dO, dht read once; every gradient written once (fp32)
    per_tok = (2 * Dk + Dv) * esz + Dv * 4 + (2 * Dk + Dv) * 4 + spec["extra"](Dk, Dv, esz)
    kbytes = float(B) * T * H * per_tok + float(B) * H * Dk * Dv * 4
    achieved = kbytes / (kms * 1e-3) / 1e9
    log(f"[bench] {args.steps} steps: {ms:.4f} ms/step wall; per call (HIP events) {kms * 1e3:.1f} us")
    res = {
        "metric": f"{spec['label']} tokens/s, T={T} d={Dk}",
        "value": B * T / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": wl, "B": B, "T": T, "H": H, "Dk": Dk, "Dv": Dv, "inputs": x["dtype"],
                   "gradients": "fp32", "stages": "forward recompute of the chunk entry states, reverse state "
                                                 "walk, per-chunk gradients; products on split bf16/fp16 "
                                                 "MFMA operands or fp32 MFMA, fp32 accumulation",
                   "buffer_sets": args.sets,
                   "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "kernel": f"{spec['fn']} (all stages)", "achieved": achieved,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "algorithmic_bytes_per_launch": kbytes, "avg_launch_us": kms * 1e3, "traffic": None},
        **timing_fields(tm),
    }
    if not args.no_cpu_baseline:
        import oracle
        # the oracle backward on one head (all of it)
        sub = [x[n + "_f64"][:1, :, :1] for n in names]
        t0 = time.perf_counter()
        getattr(oracle, spec["ref"])(*sub, None, do[:1, :, :1].astype(np.float64), dht[:1, :1].astype(np.float64),
                                     scale=x["scale"])
        dt_cpu = time.perf_counter() - t0
        res["cpu_baseline"] = {"value": T / dt_cpu, "unit": "tokens/s", "cores": 1, "kind": "oracle",
                               "sample": f"one head of the workload ({T} tokens); the oracle runs one head per "
                                         "thread, so a whole batch scales with min(cores, B*H)"}
    else:
        res["cpu_baseline"] = None
    return res


def bench_layer(args, wl):
    """The layer around the rule: prologue (short convolution, SiLU, L2 norm, gates)
    -> chunked forward -> gated RMSNorm, each kernel timed with HIP events."""
    import torch
    import gated_delta_rule_34_amd as gdn
    import gdn_inputs as gi

    dev = torch.device("cuda:0")
    x = gi.workload(wl)
    B, T, H, Dk, Dv = x["B"], x["T"], x["H"], x["Dk"], x["Dv"]
    names = ("xq", "xk", "xv", "a", "b", "wq", "wk", "wv", "A_log", "dt_bias", "z", "norm_w")
    base = {n: to_dev(x[n], dev) for n in names}
    sets = []
    for i in range(args.sets):
        s = {n: t.clone() for n, t in base.items()}
        s["o"] = torch.empty((B, T, H, Dv), dtype=torch.float32, device=dev)
        s["ht"] = torch.empty((B, H, Dk, Dv), dtype=torch.float32, device=dev)
        s["y"] = torch.empty((B, T, H, Dv), dtype=torch.bfloat16, device=dev)
        sets.append(s)
    ws = torch.empty(gdn.gdn_chunk_fwd_workspace(B, T, H, Dk, Dv, gdn.GDN_BF16), dtype=torch.uint8, device=dev)

    def step(s, ev=None):
        if ev is not None:
            ev[0].record()
        q, k, v, g, beta, _ = gdn.gdn_prologue(*[s[n] for n in names[:10]])
        if ev is not None:
            ev[1].record()
        gdn.gdn_chunk_fwd(q, k, v, g, beta, None, scale=x["scale"], workspace=ws, out=s["o"], final_state=s["ht"])
        if ev is not None:
            ev[2].record()
        gdn.gdn_gated_rmsnorm(s["o"], s["z"], s["norm_w"], eps=1e-5, out=s["y"])
        if ev is not None:
            ev[3].record()

    tm = run_timed(step, sets, args)
    ms = tm["ms_per_step"]
    # the three stages, each between events, in a pass of its own after the timed region
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    for i in range(args.steps):
        step(sets[i % len(sets)], evs[i])
    torch.cuda.synchronize()
    seg = [sum(e[j].elapsed_time(e[j + 1]) for e in evs) / args.steps for j in range(3)]
    th = float(B) * T * H
    stage_bytes = [th * (2 * (2 * Dk + Dv) * 2 + 16),                       # projections in, q k v out, gates
                   walk_algorithmic_bytes(B, T, H, Dk, Dv, 2, False) + 4.0 * th,
                   th * Dv * 8.0]                                            # o fp32, z in; y out
    knames = ["prologue_kernel", "fused_kernel", "gated_rmsnorm_kernel"]
    stages = {kn: {"avg_launch_us": t * 1e3, "algorithmic_bytes_per_launch": by,
                   "achieved_gbs": by / (t * 1e-3) / 1e9, "frac": by / (t * 1e-3) / 1e9 / HBM_PEAK_GBS}
              for kn, t, by in zip(knames, seg, stage_bytes)}
    log(f"[bench] {args.steps} steps: {ms:.4f} ms/step wall; " +
        ", ".join(f"{k} {v['avg_launch_us']:.1f} us ({v['frac']:.3f} of HBM peak)" for k, v in stages.items()))
    dom = max(range(3), key=lambda j: seg[j])
    res = {
        "metric": f"gated delta rule layer (prologue + chunked fwd + gated RMSNorm) tokens/s, T={T} d={Dk}",
        "value": B * T / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": wl, "B": B, "T": T, "H": H, "Dk": Dk, "Dv": Dv, "chunk": BT,
                   "inputs": "bf16 projections", "kernels": "prologue, fused chunked forward, gated RMSNorm",
                   "buffer_sets": args.sets, "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "kernel": knames[dom], "achieved": stages[knames[dom]]["achieved_gbs"],
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": stages[knames[dom]]["frac"],
                     "algorithmic_bytes_per_launch": stage_bytes[dom], "avg_launch_us": seg[dom] * 1e3,
                     "traffic": None},
        "stages": stages,
        **timing_fields(tm),
    }
    if not args.no_cpu_baseline:
        # the oracle's prologue and epilogue on one sequence of the workload
        import oracle
        import oracle.prologue as op
        sub = {n: x[n + "_f64"][:1] for n in ("xq", "xk", "xv", "a", "b", "z")}
        t0 = time.perf_counter()
        q, k, v, g, beta, _ = op.prologue(sub["xq"], sub["xk"], sub["xv"], sub["a"], sub["b"],
                                          *[x[n + "_f64"] for n in ("wq", "wk", "wv", "A_log", "dt_bias")])
        o, _ = oracle.gdn_fwd(q, k, v, g, beta, None, scale=x["scale"])
        op.gated_rmsnorm(o, sub["z"], x["norm_w_f64"])
        dt_cpu = time.perf_counter() - t0
        res["cpu_baseline"] = {"value": T / dt_cpu, "unit": "tokens/s", "cores": oracle.max_threads(),
                               "kind": "oracle",
                               "sample": f"1 of {B} sequences x {H} heads x {T} tokens through the oracle's "
                                         f"prologue, recurrence and epilogue, {dt_cpu:.2f} s"}
    else:
        res["cpu_baseline"] = None
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10, help="untimed steps before the settle phase")
    ap.add_argument("--workload", default="layer_bf16",
                    choices=["layer_bf16", "long_bf16", "tiny_fp32", "decode_bf16", "decode2_bf16", "gdn2_bf16",
                             "layer_bwd_bf16", "gdn2_bwd_bf16", "layer_full_bf16"])
    ap.add_argument("--sets", type=int, default=3, help="rotated input/output buffer sets")
    ap.add_argument("--settle-ms", type=float, default=SETTLE_S * 1e3,
                    help="milliseconds of back-to-back untimed steps before timing, on top of --warmup "
                         "(the GPU clock needs ~50 ms of load to settle); 0 for short profiler runs")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="after timing, run one plain device copy of MIB MiB (outside the timed region) "
                         "so that hardware byte counters can be scaled against a known size")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the path shards over (batch, head) with no exchange, see the design notes)", file=sys.stderr)
        sys.exit(2)
    if int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs as a single process on one GPU", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    if args.workload in STEPS:
        res = bench_step(args, args.workload)
    elif args.workload in BWDS:
        res = bench_bwd(args, args.workload)
    elif args.workload == "gdn2_bf16":
        res = bench_gdn2(args, args.workload)
    elif args.workload == "layer_full_bf16":
        res = bench_layer(args, args.workload)
    else:
        res = bench_gdn(args, args.workload)
    if args.copy_calibration > 0:
        n = args.copy_calibration << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        res["copy_calibration_bytes"] = n
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
