#!/usr/bin/env python3
"""Throughput of the canonical convolution on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one pass over the workload's calls (kernels only: binding, output
layout and planning run once per call before timing, and their host time is
reported as ``host_plan_us``).  Inputs are seeded synthetic tensors already in
HBM; R rotation copies of every input/output keep consecutive uses of a
buffer more than ~1 GiB of traffic apart, so the 256 MB Infinity Cache cannot
serve them.  One JSON line is printed.

Workloads
  dw_bf16_cl   (default) depthwise bf16 channels-last, N=32, C=256, 56x56,
               k in {3,5,7} x stride in {1,2}: six calls per step.  GB/s.
  dw_f32_small depthwise fp32 NCHW, 1x32x32x32, 3x3.  GB/s.
  grp_f16      grouped fp16 NCHW, 32x256x28x28 -> 512, 64 groups.  GB/s.
  dense_bf16   dense 3x3 bf16 channels-last, 64x256x56x56 -> 256.  TFLOP/s.
  convT1d_bf16 transposed 1-D bf16 NLC, 16x512x8192 -> 16383, k=4, s=2.  TFLOP/s.

``roofline`` describes the kernel with the largest average duration: its
algorithmic bytes (or FLOPs) per launch over that average, measured with HIP
events on the launch stream.  ``cpu_baseline`` times the double-precision
reference (test infrastructure) on the host cores over a bounded sample.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

METRIC = "HBM GB/s (stencil) and TFLOP/s (implicit GEMM), % of MI355X roofline"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2516.6        # dense bf16/fp16 MFMA, 256 CUs x 2048 FMA/clk x 2.4 GHz x 2
VALU_FP32_PEAK_TFLOPS = 78.6          # 256 CUs x 64 lanes x 2 FLOP/FMA x 2.4 GHz (no packed fp32)
VALU_DOT2_PEAK_TFLOPS = 157.3         # the same lanes issuing v_dot2_f32_{bf16,f16}: two FMAs each
ROOT = os.path.dirname(os.path.abspath(__file__))
PROFILES = os.path.join(ROOT, "profiles")

WORKLOADS = ("dw_bf16_cl", "dw_f32_small", "grp_f16", "dense_bf16", "convT1d_bf16")


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="dw_bf16_cl", choices=WORKLOADS)
    ap.add_argument("--rotate", type=int, default=0, help="rotation copies (0 = enough for >= 1 GiB)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="target CPU work for the baseline")
    ap.add_argument("--probe-copy", type=int, default=0, metavar="MIB",
                    help="instead of a workload, time a plain device copy of MIB mebibytes (the "
                         "measured bandwidth ceiling, and the reference for HBM byte counters)")
    return ap.parse_args()


def copy_probe(mib, steps, warmup):
    """A plain device-to-device copy of a known size: achieved GB/s counts the
    bytes read plus the bytes written."""
    import torch
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(warmup):
        dst.copy_(src)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(steps):
        dst.copy_(src)
    ev1.record()
    torch.cuda.synchronize()
    us = ev0.elapsed_time(ev1) * 1e3 / steps
    moved = 2 * n * 4
    print(json.dumps({"probe": "copy", "bytes_per_launch": moved, "read_bytes": n * 4, "write_bytes": n * 4,
                      "avg_us": round(us, 2), "GBps": round(moved / us / 1e3, 1)}), flush=True)


def workload_calls(name):
    from depthwise_stencil_implicit_amd import synth
    if name == "dw_bf16_cl":
        return synth.depthwise_bf16_cl_all(), "GB/s"
    if name == "dw_f32_small":
        return [synth.depthwise_f32_small()], "GB/s"
    if name == "grp_f16":
        return [synth.grouped_f16()], "GB/s"
    if name == "dense_bf16":
        return [synth.dense_bf16_cl()], "TFLOP/s"
    return [synth.transposed_bf16_nlc()], "TFLOP/s"


def expand(wl):
    r = len(wl.x_shape) - 2
    ex = lambda v: tuple(v) * r if len(v) == 1 else tuple(v)
    return dict(transposed=wl.transposed, groups=wl.groups, stride=ex(wl.stride),
                padding_before=ex(wl.padding_before), padding_after=ex(wl.padding_after),
                dilation=ex(wl.dilation), output_padding=ex(wl.output_padding))


def kernel_source_sha(kernel_name):
    files = {"dw_cl": "k_dwcl.hip", "plane": "k_plane.hip", "grp": "k_grp.hip", "reduce": "k_reduce.hip",
             "igemm": "k_igemm.hip", "igemm_t": "k_igemm.hip"}
    h = hashlib.sha256()
    for f in (files.get(kernel_name, ""), "dev_common.h"):
        p = os.path.join(ROOT, "depthwise_stencil_implicit_amd", "csrc", f)
        if os.path.isfile(p):
            h.update(open(p, "rb").read())
    return h.hexdigest()[:16]


def measured_traffic(kernel_name, call_name):
    """HBM bytes per launch from a committed rocprofv3 counter summary, or
    None when there is none or the kernel source changed since."""
    path = os.path.join(PROFILES, f"traffic_{kernel_name}_{call_name}.txt")
    if not os.path.isfile(path):
        return None
    fields = {}
    for ln in open(path):
        m = re.match(r"^(\w+):\s*(\S+)", ln)
        if m:
            fields[m.group(1)] = m.group(2)
    if fields.get("source_sha") != kernel_source_sha(kernel_name):
        return None
    try:
        return float(fields["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(calls, unit, target_s):
    """The reference on a bounded sample of the workload: the leading images
    of each call, sized from a one-image timing so the whole sample takes about
    ``target_s``; when even the full batch is quicker, the full batch is run
    repeatedly until ``target_s`` has passed."""
    import oracle
    from depthwise_stencil_implicit_amd import synth
    cores = len(os.sched_getaffinity(0))
    f = lambda t: None if t is None else t.double().contiguous().numpy()
    plan = []
    for wl in calls:
        one = wl.with_batch(1)
        x, w, b = synth.make_inputs(one)
        t0 = time.perf_counter()
        oracle.conv(f(x), f(w), f(b), nthreads=cores, **expand(one))
        t_one = time.perf_counter() - t0
        n = max(1, min(wl.x_shape[0], int(target_s / len(calls) / max(t_one, 1e-6))))
        sub = wl.with_batch(n)
        plan.append((sub, synth.make_inputs(sub), call_work(sub, unit)))
    total_t, total_work, rounds = 0.0, 0.0, 0
    while rounds == 0 or total_t < 0.5 * target_s:
        for sub, (x, w, b), work in plan:
            t0 = time.perf_counter()
            oracle.conv(f(x), f(w), f(b), nthreads=cores, **expand(sub))
            total_t += time.perf_counter() - t0
            total_work += work
        rounds += 1
    value = total_work / total_t / (1e9 if unit == "GB/s" else 1e12)
    samples = ", ".join(f"{sub.name.split('@')[0]}:N={sub.x_shape[0]}" for sub, _, _ in plan)
    return {"value": round(value, 4), "unit": unit, "cores": int(oracle.max_threads()), "kind": "oracle",
            "sample": f"double-precision reference over {samples}, {rounds} pass(es), {total_t:.1f} s wall"}


def wl0_dtype(calls):
    return calls[0].dtype


def call_work(wl, unit):
    """Algorithmic bytes or FLOPs of one call, from the library's plan."""
    import torch
    from depthwise_stencil_implicit_amd import api, synth
    dt = synth.DTYPES[wl.dtype]
    x = torch.empty(wl.x_shape, dtype=dt)
    if wl.channels_last:
        x = synth.channels_last_copy(x)
    w = torch.empty(wl.w_shape, dtype=dt)
    c_out = wl.w_shape[1] * wl.groups if wl.transposed else wl.w_shape[0]
    b = torch.empty((c_out,), dtype=dt) if wl.has_bias else None
    kw = expand(wl)
    args = api.make_args(transposed=kw["transposed"], groups=kw["groups"], stride=kw["stride"],
                         padding_before=kw["padding_before"], padding_after=kw["padding_after"],
                         dilation=kw["dilation"],
                         output_padding=kw["output_padding"] if kw["transposed"] else None)
    p = api.Prepared(x, w, b, args).plan
    return float(p.bytes if unit == "GB/s" else p.flops)


def main():
    a = parse()
    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; --gpus must be 1 "
                                   "(multi-GPU sharding is described, not built)"}), flush=True)
        sys.exit(2)
    import torch
    from depthwise_stencil_implicit_amd import api, synth

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}), flush=True)
        sys.exit(1)
    dev = torch.device("cuda:0")
    if a.probe_copy:
        copy_probe(a.probe_copy, a.steps, a.warmup)
        return
    calls, unit = workload_calls(a.workload)

    # ---- bind / out_shape / plan once per call (host time reported) ----
    preps, host_us = [], []
    per_call_bytes = []
    for wl in calls:
        x, w, b = synth.make_inputs(wl)
        kw = expand(wl)
        t0 = time.perf_counter()
        args = api.make_args(transposed=kw["transposed"], groups=kw["groups"], stride=kw["stride"],
                             padding_before=kw["padding_before"], padding_after=kw["padding_after"],
                             dilation=kw["dilation"],
                             output_padding=kw["output_padding"] if kw["transposed"] else None)
        p = api.Prepared(x, w, b, args)
        host_us.append((time.perf_counter() - t0) * 1e6)
        footprint = (x.numel() + w.numel() + (b.numel() if b is not None else 0)) * x.element_size() + \
            int(torch.Size(p.sizes).numel()) * x.element_size()
        per_call_bytes.append(footprint)
        preps.append((wl, p, (x, w, b)))

    # ---- device buffers, rotated so a buffer's reuse is >= ~1 GiB apart ----
    step_bytes = sum(per_call_bytes)
    R = a.rotate or max(2, -(-(1 << 30) // max(step_bytes, 1)) + 1)
    R = min(R, 64)
    sets = []
    for (wl, p, (x, w, b)) in preps:
        rs = []
        for _ in range(R):
            xd = torch.empty_strided(x.shape, x.stride(), dtype=x.dtype, device=dev)
            xd.copy_(x)
            wd, bd = w.to(dev), (b.to(dev) if b is not None else None)
            yd = p.empty_output(dev)
            ws = p.workspace(dev)
            rs.append((xd, wd, bd, yd, ws))
        sets.append(rs)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    sptr = stream.cuda_stream

    def step(i, evs=None):
        r = i % R
        for c, (wl, p, _) in enumerate(preps):
            xd, wd, bd, yd, ws = sets[c][r]
            if evs is not None:
                evs[c][0].record(stream)
            p.run(xd, wd, bd, yd, ws, sptr)
            if evs is not None:
                evs[c][1].record(stream)

    for i in range(a.warmup):
        step(i)
    torch.cuda.synchronize()

    # ---- timed region: exactly K steps, synchronised on both sides ----
    t0 = time.perf_counter()
    for i in range(a.steps):
        step(a.warmup + i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / a.steps

    # ---- per-kernel durations with events on the launch stream ----
    ev = [[[torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)]
           for _ in preps] for _ in range(a.steps)]
    for i in range(a.steps):
        step(a.warmup + a.steps + i, ev[i])
    torch.cuda.synchronize()
    per_call = []
    for c, (wl, p, _) in enumerate(preps):
        durs = sorted(ev[i][c][0].elapsed_time(ev[i][c][1]) for i in range(a.steps))
        avg_us = 1e3 * sum(durs) / len(durs)
        med_us = 1e3 * durs[len(durs) // 2]
        kname = api.kernel_name(p.plan.kernel)
        flops, nbytes = float(p.plan.flops), float(p.plan.bytes)
        per_call.append(dict(call=wl.name, kernel=kname, variant=int(p.plan.variant), avg_us=round(avg_us, 2),
                             median_us=round(med_us, 2),
                             GBps=round(nbytes / avg_us / 1e3, 1), TFLOPs=round(flops / avg_us / 1e6, 2),
                             bytes=int(nbytes), flops=int(flops), host_plan_us=round(host_us[c], 1)))

    total_bytes = sum(c["bytes"] for c in per_call)
    total_flops = sum(c["flops"] for c in per_call)
    if unit == "GB/s":
        value = total_bytes / (ms_per_step * 1e-3) / 1e9
    else:
        value = total_flops / (ms_per_step * 1e-3) / 1e12

    # ---- roofline of the dominant kernel ----
    dom = max(per_call, key=lambda c: c["avg_us"])
    ai = dom["flops"] / dom["bytes"]
    # The 16-bit stencils (dw_cl, grp) multiply through packed dot2, two FMAs
    # per lane and instruction; every other vector path issues one FMA.  The
    # grouped kernel's matrix-core schedule (plan variant 1) multiplies on
    # MFMA, whose ridge (~315 FLOP/B) puts every stencil on the HBM side.
    valu_peak = VALU_DOT2_PEAK_TFLOPS if (dom["kernel"] in ("dw_cl", "grp") and wl0_dtype(calls) != "f32") \
        else VALU_FP32_PEAK_TFLOPS
    if dom["kernel"] == "grp" and dom["variant"] == 1:
        valu_peak = MFMA_BF16_PEAK_TFLOPS
    if dom["kernel"] in ("igemm", "igemm_t"):
        roof = dict(bound="mfma", achieved=dom["TFLOPs"], peak=MFMA_BF16_PEAK_TFLOPS, unit="TFLOP/s")
    elif ai > valu_peak * 1e12 / (HBM_PEAK_GBS * 1e9):
        roof = dict(bound="alu", achieved=dom["TFLOPs"], peak=valu_peak, unit="TFLOP/s")
    else:
        roof = dict(bound="hbm", achieved=dom["GBps"], peak=HBM_PEAK_GBS, unit="GB/s")
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    roof["traffic"] = measured_traffic(dom["kernel"], dom["call"])
    roof["kernel"] = dom["kernel"]
    roof["call"] = dom["call"]
    roof["avg_us"] = dom["avg_us"]

    wl0 = calls[0]
    config = {"workload": a.workload, "calls": [c.name for c in calls], "dtype": wl0.dtype,
              "rotation_sets": R, "timing": "wall clock over K steps; per-kernel HIP events"}
    out = {"metric": METRIC, "value": round(value, 3), "unit": unit, "n_gpus": 1, "steps": a.steps,
           "warmup": a.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": wl0.dtype, "data": "synthetic",
           "config": config, "roofline": roof, "per_call": per_call}
    if a.no_cpu_baseline:
        out["cpu_baseline"] = None
    else:
        out["cpu_baseline"] = cpu_baseline(calls, unit, a.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
