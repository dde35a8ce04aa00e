#!/usr/bin/env python3
"""Throughput of the canonical convolution on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
    python bench.py --probe-copy MIB | --probe-mfma | --probe-valu | --probe-lds
    python bench.py --backward     gradients (dx, dw, db) of every call of the default run

A step is one pass over the workload's calls (kernels only: binding, output
layout and planning run once per call before timing, and their host time is
reported as ``host_plan_us``).  Inputs are seeded synthetic tensors already in
HBM; R rotation copies of every input/output keep consecutive uses of a
buffer more than ~1 GiB of traffic apart, so the 256 MB Infinity Cache cannot
serve them.  ``--graph`` captures each rotation set's step once in a HIP graph
and times graph replays instead of eager launches (the library's launches
are capturable: kernels only).  One JSON line is printed.

Workloads
  all          (default) every measured workload below in one step: the
               depthwise fp32 call, the six depthwise bf16 calls, the grouped
               call, the dense call and the transposed call.  ``value`` is the
               step's percentage of the MI355X roofline: the sum over the
               calls of their time at the roofline (algorithmic bytes at
               8 TB/s or algorithmic FLOPs at the relevant compute peak,
               whichever is longer) over the measured step time.  Each
               workload also gets its own row (GB/s or TFLOP/s, fraction).
  dw_bf16_cl   depthwise bf16 channels-last, N=32, C=256, 56x56,
               k in {3,5,7} x stride in {1,2}: six calls per step.  GB/s.
  dw_f32_small depthwise fp32 NCHW, 1x32x32x32, 3x3.  GB/s.
  grp_f16      grouped fp16 NCHW, 32x256x28x28 -> 512, 64 groups.  GB/s.
  dense_bf16   dense 3x3 bf16 channels-last, 64x256x56x56 -> 256.  TFLOP/s.
  convT1d_bf16 transposed 1-D bf16 NLC, 16x512x8192 -> 16383, k=4, s=2.  TFLOP/s.
  edges        calls at the edges of the fast paths, each its own row (not
               part of ``all``): depthwise 9x9 and stride 3, a channel
               multiplier of 2, 1-D depthwise, 3-D dense, 2-D transposed.
               ``value`` as for ``all``.

``roofline`` describes the call with the largest average duration: its
algorithmic bytes (or FLOPs) per launch over that average, measured with HIP
events on the launch stream around eager launches of each call.  ``cpu_baseline`` times the double-precision
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
MFMA_F32_PEAK_TFLOPS = 157.3          # dense fp32 MFMA
VALU_FP32_PEAK_TFLOPS = 157.3         # published fp32 vector peak; v_fmac_f32 issues a wave in ~2 clocks (probe)
VALU_DOT2_PEAK_TFLOPS = 157.3         # v_dot2_f32_{bf16,f16}: two FMAs per lane, a wave in 4 clocks
ROOT = os.path.dirname(os.path.abspath(__file__))
PROFILES = os.path.join(ROOT, "profiles")

WORKLOADS = ("all", "dw_f32_small", "dw_bf16_cl", "grp_f16", "dense_bf16", "convT1d_bf16", "edges")
# The five measured workloads (the default run), and the domain-edge calls.
MEASURED = ("dw_f32_small", "dw_bf16_cl", "grp_f16", "dense_bf16", "convT1d_bf16")
META = ("all", "edges")
UNITS = {"dw_f32_small": "GB/s", "dw_bf16_cl": "GB/s", "grp_f16": "GB/s", "dense_bf16": "TFLOP/s",
         "convT1d_bf16": "TFLOP/s"}


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="all", choices=WORKLOADS)
    ap.add_argument("--rotate", type=int, default=0, help="rotation copies (0 = enough for >= 1 GiB)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--rule", action="store_true",
                    help="run the planner's rule-based schedules (default: time every candidate schedule of each "
                         "call once while planning, conv_tune, and run the fastest)")
    ap.add_argument("--cpu-seconds", type=float, default=20.0, help="target CPU work for the baseline")
    ap.add_argument("--graph", action="store_true",
                    help="capture each rotation set's step once in a HIP graph and time graph replays (default: "
                         "eager launches; on the default workload both measure the same step time)")
    ap.add_argument("--backward", action="store_true",
                    help="instead of the forward step, time conv_run_backward (dx, dw and db) for every call of "
                         "the default run, one JSON line with a row per call")
    ap.add_argument("--probe-copy", type=int, default=0, metavar="MIB",
                    help="instead of a workload, time a plain device copy of MIB mebibytes (the "
                         "measured bandwidth ceiling, and the reference for HBM byte counters)")
    ap.add_argument("--probe-mfma", action="store_true",
                    help="instead of a workload, time a kernel of independent bf16 MFMAs (the "
                         "measured matrix-core ceiling)")
    ap.add_argument("--probe-valu", action="store_true",
                    help="instead of a workload, time kernels of independent vector bf16 dot2 and fp32 FMA "
                         "instructions (the measured vector-ALU ceilings)")
    ap.add_argument("--probe-lds", action="store_true",
                    help="instead of a workload, time a kernel of conflict-free 16-byte LDS reads")
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


def backward_bench(steps, warmup):
    """Gradients of every call of the default run: conv_run_backward with dx,
    dw and db together, averaged over HIP events on the launch stream (warm
    buffers, no rotation).  A call's time at the roofline is the longer of its
    algorithmic bytes (the plan's dx + dw + db bytes) at 8 TB/s and its FLOPs
    (dx and dw each count as many as the forward call) at the matrix-core peak
    of its dtype (the vector peak for fp32)."""
    import torch
    from depthwise_stencil_implicit_amd import api, synth
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    rows = []
    for wname, wl in workload_calls("all"):
        x, w, b = synth.make_inputs(wl, device="cuda")
        args = make_args(wl)
        y = api.Prepared(x, w, b, args).empty_output(dev)
        g = torch.Generator(device="cuda").manual_seed(wl.seed + 1)
        gy = torch.randn(y.shape, generator=g, device=dev, dtype=torch.float32).to(y.dtype)
        gy = torch.empty_strided(y.shape, y.stride(), dtype=y.dtype, device=dev).copy_(gy)
        try:
            pb = api.PreparedBackward(x, w, gy, args)
        except api.ConvError as e:
            rows.append({"workload": wname, "call": wl.name, "error": str(e)})
            continue
        dx, dw, db = pb.outputs(dev)
        ws = pb.workspace(dev)
        for _ in range(warmup):
            pb.run(x, w, gy, dx, dw, db, ws, stream.cuda_stream)
        torch.cuda.synchronize()
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ev0.record(stream)
        for _ in range(steps):
            pb.run(x, w, gy, dx, dw, db, ws, stream.cuda_stream)
        ev1.record(stream)
        torch.cuda.synchronize()
        us = ev0.elapsed_time(ev1) * 1e3 / steps
        fl, by = int(sum(pb.plan.flops)), int(sum(pb.plan.bytes))
        peak = VALU_FP32_PEAK_TFLOPS if wl.dtype == "f32" else MFMA_BF16_PEAK_TFLOPS
        t_mem, t_cmp = by / (HBM_PEAK_GBS * 1e3), fl / (peak * 1e6)
        bound = "mfma" if t_cmp > t_mem and wl.dtype != "f32" else ("alu" if t_cmp > t_mem else "hbm")
        rows.append({"workload": wname, "call": wl.name, "dgrad_kernel": api.kernel_name(pb.plan.dgrad.kernel),
                     "avg_us": round(us, 2), "gflop": round(fl / 1e9, 3), "mb": round(by / 1e6, 2),
                     "TFLOPs": round(fl / us / 1e6, 2), "GBps": round(by / us / 1e3, 1), "bound": bound,
                     "frac": round(max(t_mem, t_cmp) / us, 4)})
        print(json.dumps(rows[-1]), file=sys.stderr, flush=True)
        del x, w, b, y, gy, dx, dw, db, ws, pb
        torch.cuda.empty_cache()
    print(json.dumps({"mode": "backward", "steps": steps, "warmup": warmup, "data": "synthetic",
                      "per_call": rows}), flush=True)


def unit_probe(kind, steps, warmup):
    """MFMA or vector-ALU issue rate, or LDS read bandwidth, from the probe
    library's kernels (8 workgroups of 256 threads per CU, 256 CUs).  The MFMA
    and vector probes also read the shader clock against the 100 MHz real-time
    counter inside their loops, which gives the clock the units ran at."""
    import ctypes
    import torch
    from depthwise_stencil_implicit_amd import build
    if not os.path.exists(build.PROBE_LIB):
        raise SystemExit(f"{build.PROBE_LIB} is missing: run the build first")
    lib = ctypes.CDLL(build.PROBE_LIB)
    blocks = 256 * 8
    out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda:0")
    clk = torch.zeros(blocks * 2, dtype=torch.int64, device="cuda:0")
    stream = torch.cuda.current_stream()
    if kind == "mfma":
        lib.probe_mfma.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                   ctypes.c_void_p]
        lib.probe_mfma.restype = ctypes.c_int
        iters = 4096
        shapes = [("mfma_bf16_16x16x32", 0, 8 * 16 * 16 * 32 * 2), ("mfma_bf16_32x32x16", 1, 4 * 32 * 32 * 16 * 2)]
        for name, big, flop_per_round in shapes:
            fn = lambda: lib.probe_mfma(out.data_ptr(), clk.data_ptr(), blocks, iters, big, stream.cuda_stream)
            for _ in range(warmup):
                assert fn() == 0
            torch.cuda.synchronize()
            ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            ev0.record(stream)
            for _ in range(steps):
                assert fn() == 0
            ev1.record(stream)
            torch.cuda.synchronize()
            us = ev0.elapsed_time(ev1) * 1e3 / steps
            flops = blocks * 4 * iters * flop_per_round
            rate = flops / us / 1e6
            c = clk.view(-1, 2).double()
            mhz = float((c[:, 0] / c[:, 1].clamp(min=1)).median()) * 100.0
            cyc = float(c[:, 0].median()) / iters / (8 if not big else 4)
            print(json.dumps({"probe": name, "flops_per_launch": flops, "avg_us": round(us, 2),
                              "TFLOPs": round(rate, 1), "peak_TFLOPs": MFMA_BF16_PEAK_TFLOPS,
                              "frac": round(rate / MFMA_BF16_PEAK_TFLOPS, 4), "shader_clock_MHz": round(mhz),
                              "clocks_per_mfma_per_wave": round(cyc, 2)}), flush=True)
    elif kind == "valu":
        lib.probe_valu.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                   ctypes.c_void_p]
        lib.probe_valu.restype = ctypes.c_int
        iters = 8192
        # FLOPs per lane per round: 8 instructions of 2 products (dot2) or 1 (FMA), 2 FLOP each.
        shapes = [("valu_dot2_f32_bf16", 0, 8 * 2 * 2, VALU_DOT2_PEAK_TFLOPS),
                  ("valu_fma_f32", 1, 8 * 1 * 2, VALU_FP32_PEAK_TFLOPS),
                  ("valu_dot2c_bf16 operands in one register bank", 2, 8 * 2 * 2, VALU_DOT2_PEAK_TFLOPS),
                  ("valu_dot2c_bf16 operands in three banks", 3, 8 * 2 * 2, VALU_DOT2_PEAK_TFLOPS),
                  ("valu_dot2c_bf16 accumulator and second source in one bank", 4, 8 * 2 * 2,
                   VALU_DOT2_PEAK_TFLOPS)]
        for name, kind_id, flop_per_round, peak in shapes:
            fn = lambda: lib.probe_valu(out.data_ptr(), clk.data_ptr(), blocks, iters, kind_id, stream.cuda_stream)
            for _ in range(warmup):
                assert fn() == 0
            torch.cuda.synchronize()
            ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            ev0.record(stream)
            for _ in range(steps):
                assert fn() == 0
            ev1.record(stream)
            torch.cuda.synchronize()
            us = ev0.elapsed_time(ev1) * 1e3 / steps
            flops = blocks * 256 * iters * flop_per_round
            rate = flops / us / 1e6
            c = clk.view(-1, 2).double()
            mhz = float((c[:, 0] / c[:, 1].clamp(min=1)).median()) * 100.0
            cyc = float(c[:, 0].median()) / iters / 8
            print(json.dumps({"probe": name, "flops_per_launch": flops, "avg_us": round(us, 2),
                              "TFLOPs": round(rate, 1), "peak_TFLOPs": peak, "frac": round(rate / peak, 4),
                              "shader_clock_MHz": round(mhz), "clocks_per_instr_per_wave": round(cyc, 2)}),
                  flush=True)
    else:
        lib.probe_lds.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
        lib.probe_lds.restype = ctypes.c_int
        iters = 2048
        fn = lambda: lib.probe_lds(out.data_ptr(), blocks, iters, stream.cuda_stream)
        for _ in range(warmup):
            assert fn() == 0
        torch.cuda.synchronize()
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ev0.record(stream)
        for _ in range(steps):
            assert fn() == 0
        ev1.record(stream)
        torch.cuda.synchronize()
        us = ev0.elapsed_time(ev1) * 1e3 / steps
        nbytes = blocks * 256 * iters * 8 * 16
        rate = nbytes / us / 1e6
        print(json.dumps({"probe": "lds_read_b128", "bytes_per_launch": nbytes, "avg_us": round(us, 2),
                          "TBps": round(rate, 2),
                          "bytes_per_clk_per_cu_at_2.4GHz": round(nbytes / (us * 1e-6) / 2.4e9 / 256, 1)}),
              flush=True)


def workload_calls(name):
    """[(workload name, call)] for a bench workload."""
    from depthwise_stencil_implicit_amd import synth
    table = {"dw_f32_small": [synth.depthwise_f32_small()], "dw_bf16_cl": synth.depthwise_bf16_cl_all(),
             "grp_f16": [synth.grouped_f16()], "dense_bf16": [synth.dense_bf16_cl()],
             "convT1d_bf16": [synth.transposed_bf16_nlc()]}
    if name == "edges":
        # Each edge call is a workload of its own, in the unit of its bound.
        return [(wl.name, wl) for wl in synth.domain_edge_workloads()]
    names = list(MEASURED) if name == "all" else [name]
    return [(n, wl) for n in names for wl in table[n]]


def expand(wl):
    r = len(wl.x_shape) - 2
    ex = lambda v: tuple(v) * r if len(v) == 1 else tuple(v)
    return dict(transposed=wl.transposed, groups=wl.groups, stride=ex(wl.stride),
                padding_before=ex(wl.padding_before), padding_after=ex(wl.padding_after),
                dilation=ex(wl.dilation), output_padding=ex(wl.output_padding))


def kernel_source_sha(kernel_name):
    files = {"dw_cl": ("k_dwcl.hip",), "plane": ("k_plane.hip",), "grp": ("k_grp.hip",),
             "reduce": ("k_reduce.hip",), "igemm": ("k_igemm.hip",), "igemm_t": ("k_igemm.hip", "k_igemm_t1.hip")}
    h = hashlib.sha256()
    for f in files.get(kernel_name, ()) + ("dev_common.h",):
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


def make_args(wl):
    from depthwise_stencil_implicit_amd import api
    kw = expand(wl)
    return api.make_args(transposed=kw["transposed"], groups=kw["groups"], stride=kw["stride"],
                         padding_before=kw["padding_before"], padding_after=kw["padding_after"],
                         dilation=kw["dilation"], output_padding=kw["output_padding"] if kw["transposed"] else None)


def call_plan(wl):
    """The library's plan of a call (host only), for its algorithmic units."""
    import torch
    from depthwise_stencil_implicit_amd import api, synth
    dt = synth.DTYPES[wl.dtype]
    x = torch.empty(wl.x_shape, dtype=dt)
    if wl.channels_last:
        x = synth.channels_last_copy(x)
    w = torch.empty(wl.w_shape, dtype=dt)
    c_out = wl.w_shape[1] * wl.groups if wl.transposed else wl.w_shape[0]
    b = torch.empty((c_out,), dtype=dt) if wl.has_bias else None
    return api.Prepared(x, w, b, make_args(wl)).plan


def roof_of(kernel, variant, dtype, flops, nbytes):
    """(bound, peak, time at the roofline in us) of one call: the longer of
    its algorithmic bytes at 8 TB/s and its FLOPs at the compute peak of the
    units the kernel multiplies on."""
    if kernel in ("igemm", "igemm_t") or (kernel == "grp" and variant == 1):
        cpeak, cbound = (MFMA_F32_PEAK_TFLOPS if dtype == "f32" else MFMA_BF16_PEAK_TFLOPS), "mfma"
    elif dtype == "f32":
        cpeak, cbound = VALU_FP32_PEAK_TFLOPS, "alu"
    else:
        cpeak, cbound = VALU_DOT2_PEAK_TFLOPS, "alu"
    t_mem = nbytes / (HBM_PEAK_GBS * 1e3)          # us
    t_cmp = flops / (cpeak * 1e6)                    # us
    if kernel in ("igemm", "igemm_t") or t_cmp > t_mem:
        return cbound, cpeak, max(t_cmp, t_mem)
    return "hbm", HBM_PEAK_GBS, t_mem


def unit_of(wname, plan):
    """GB/s or TFLOP/s: a measured workload's own unit, else the unit of the
    call's bound."""
    if wname in UNITS:
        return UNITS[wname]
    from depthwise_stencil_implicit_amd import api
    bound, _, _ = roof_of(api.kernel_name(plan.kernel), int(plan.variant), "bf16", float(plan.flops),
                          float(plan.bytes))
    return "GB/s" if bound == "hbm" else "TFLOP/s"


def cpu_model():
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(calls, target_s, headline_pct):
    """The reference on a bounded sample of the workload: the leading images
    of each call, sized from a one-image timing so the whole sample takes
    about ``target_s``; when even the full batch is quicker, the full batch is
    run repeatedly.  Reported in the headline's unit (percent of the GPU's
    roofline for the sampled calls) and per workload in GB/s or TFLOP/s."""
    import oracle
    from depthwise_stencil_implicit_amd import api, synth
    cores = len(os.sched_getaffinity(0))
    f = lambda t: None if t is None else t.double().contiguous().numpy()
    plan = []
    for wname, wl in calls:
        one = wl.with_batch(1)
        x, w, b = synth.make_inputs(one)
        t0 = time.perf_counter()
        oracle.conv(f(x), f(w), f(b), nthreads=cores, **expand(one))
        t_one = time.perf_counter() - t0
        n = max(1, min(wl.x_shape[0], int(target_s / len(calls) / max(t_one, 1e-6))))
        sub = wl.with_batch(n)
        p = call_plan(sub)
        plan.append((wname, sub, synth.make_inputs(sub), p))
    total_t, rounds = 0.0, 0
    per = {}
    while rounds == 0 or total_t < 0.5 * target_s:
        for wname, sub, (x, w, b), p in plan:
            t0 = time.perf_counter()
            oracle.conv(f(x), f(w), f(b), nthreads=cores, **expand(sub))
            dt = time.perf_counter() - t0
            total_t += dt
            _, _, t_roof = roof_of(api.kernel_name(p.kernel), int(p.variant), sub.dtype, float(p.flops),
                                   float(p.bytes))
            e = per.setdefault(wname, [0.0, 0.0, 0.0, 0.0])
            e[0] += dt
            e[1] += float(p.bytes)
            e[2] += float(p.flops)
            e[3] += t_roof * 1e-6
        rounds += 1
    rows = []
    for wname, (t, nb, fl, tr) in per.items():
        unit = unit_of(wname, next(p for n, _, _, p in plan if n == wname))
        rows.append({"workload": wname, "unit": unit,
                     "value": round(nb / t / 1e9 if unit == "GB/s" else fl / t / 1e12, 5)})
    pct = 100.0 * sum(e[3] for e in per.values()) / sum(e[0] for e in per.values())
    samples = ", ".join(f"{sub.name.split('@')[0]}:N={sub.x_shape[0]}" for _, sub, _, _ in plan)
    out = {"value": round(pct, 6), "unit": "% of MI355X roofline", "cores": int(oracle.max_threads()),
           "kind": "oracle", "cpu_model": cpu_model(), "per_workload": rows,
           "sample": f"double-precision reference over {samples}, {rounds} pass(es), {total_t:.1f} s wall"}
    if headline_pct is not None and pct > 0:
        out["gpu_over_cpu"] = round(headline_pct / pct, 1)
    return out


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
    if a.backward:
        backward_bench(a.steps, a.warmup)
        return
    if a.probe_mfma or a.probe_valu or a.probe_lds:
        unit_probe("mfma" if a.probe_mfma else ("valu" if a.probe_valu else "lds"), a.steps, a.warmup)
        return
    calls = workload_calls(a.workload)

    # ---- bind / out_shape / plan once per call (host time reported) ----
    preps, host_us, per_call_bytes = [], [], []
    for wname, wl in calls:
        x, w, b = synth.make_inputs(wl)
        t0 = time.perf_counter()
        p = api.Prepared(x, w, b, make_args(wl))
        if not a.rule:
            xd, wd = x.to(dev), w.to(dev)          # .to keeps x's strides
            p.tune(xd, wd, b.to(dev) if b is not None else None, reps=3)
            del xd, wd
        host_us.append((time.perf_counter() - t0) * 1e6)
        footprint = (x.numel() + w.numel() + (b.numel() if b is not None else 0)) * x.element_size() + \
            int(torch.Size(p.sizes).numel()) * x.element_size()
        per_call_bytes.append(footprint)
        preps.append((wname, wl, p, (x, w, b)))

    # ---- device buffers, rotated so a buffer's reuse is >= ~1 GiB apart ----
    step_bytes = sum(per_call_bytes)
    R = a.rotate or max(2, -(-(1 << 30) // max(step_bytes, 1)) + 1)
    R = min(R, 64)
    sets = []
    for (_, wl, p, (x, w, b)) in preps:
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

    def launch(r, sp, evs=None, st=None):
        for c, (_, wl, p, _) in enumerate(preps):
            xd, wd, bd, yd, ws = sets[c][r]
            if evs is not None:
                evs[c][0].record(st)
            p.run(xd, wd, bd, yd, ws, sp)
            if evs is not None:
                evs[c][1].record(st)

    def step(i, evs=None):
        launch(i % R, sptr, evs, stream)

    for i in range(a.warmup):
        step(i)
    torch.cuda.synchronize()

    # ---- the step as HIP graphs: every call of rotation set r captured once
    # (the library launches only kernels, no memsets or allocations) ----
    graphs = []
    if a.graph:
        cs = torch.cuda.Stream(dev)
        for r in range(R):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=cs):
                launch(r, torch.cuda.current_stream(dev).cuda_stream)
            graphs.append(g)
        for i in range(a.warmup):
            graphs[i % R].replay()
        torch.cuda.synchronize()

    # ---- timed region: exactly K steps, synchronised on both sides ----
    t0 = time.perf_counter()
    for i in range(a.steps):
        if graphs:
            graphs[(a.warmup + i) % R].replay()
        else:
            step(a.warmup + i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / a.steps

    # ---- per-call durations with events on the launch stream ----
    ev = [[[torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)]
           for _ in preps] for _ in range(a.steps)]
    for i in range(a.steps):
        step(a.warmup + a.steps + i, ev[i])
    torch.cuda.synchronize()
    per_call = []
    for c, (wname, wl, p, _) in enumerate(preps):
        durs = sorted(ev[i][c][0].elapsed_time(ev[i][c][1]) for i in range(a.steps))
        avg_us = 1e3 * sum(durs) / len(durs)
        med_us = 1e3 * durs[len(durs) // 2]
        kname = api.kernel_name(p.plan.kernel)
        flops, nbytes = float(p.plan.flops), float(p.plan.bytes)
        bound, peak, t_roof = roof_of(kname, int(p.plan.variant), wl.dtype, flops, nbytes)
        achieved = nbytes / avg_us / 1e3 if bound == "hbm" else flops / avg_us / 1e6
        per_call.append(dict(workload=wname, call=wl.name, kernel=kname, variant=int(p.plan.variant),
                             avg_us=round(avg_us, 2), median_us=round(med_us, 2),
                             GBps=round(nbytes / avg_us / 1e3, 1), TFLOPs=round(flops / avg_us / 1e6, 2),
                             bytes=int(nbytes), flops=int(flops), bound=bound, roof_us=round(t_roof, 3),
                             frac=round(achieved / peak, 4), host_plan_us=round(host_us[c], 1)))

    # ---- per-workload rows and the headline ----
    rows = []
    for wname in dict.fromkeys(c["workload"] for c in per_call):
        cs = [c for c in per_call if c["workload"] == wname]
        t = sum(c["avg_us"] for c in cs)
        unit = UNITS.get(wname) or ("GB/s" if cs[0]["bound"] == "hbm" else "TFLOP/s")
        val = sum(c["bytes"] for c in cs) / t / 1e3 if unit == "GB/s" else sum(c["flops"] for c in cs) / t / 1e6
        rows.append({"workload": wname, "calls": len(cs), "unit": unit, "value": round(val, 2),
                     "us": round(t, 2), "roof_us": round(sum(c["roof_us"] for c in cs), 3),
                     "frac_of_roofline": round(sum(c["roof_us"] for c in cs) / t, 4)})
    roof_total_us = sum(c["roof_us"] for c in per_call)
    if a.workload in META:
        value, unit = 100.0 * roof_total_us / (ms_per_step * 1e3), "% of MI355X roofline"
    else:
        unit = UNITS[a.workload]
        tot = sum(c["bytes"] for c in per_call) if unit == "GB/s" else sum(c["flops"] for c in per_call)
        value = tot / (ms_per_step * 1e-3) / (1e9 if unit == "GB/s" else 1e12)

    # ---- roofline of the dominant call ----
    dom = max(per_call, key=lambda c: c["avg_us"])
    if dom["bound"] == "hbm":
        roof = dict(bound="hbm", achieved=dom["GBps"], peak=HBM_PEAK_GBS, unit="GB/s")
    else:
        _, peak, _ = roof_of(dom["kernel"], dom["variant"], next(wl.dtype for _, wl, _, _ in preps
                                                                   if wl.name == dom["call"]),
                             dom["flops"], dom["bytes"])
        roof = dict(bound=dom["bound"], achieved=dom["TFLOPs"], peak=peak, unit="TFLOP/s")
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    roof["traffic"] = measured_traffic(dom["kernel"], dom["call"])
    roof["kernel"] = dom["kernel"]
    roof["call"] = dom["call"]
    roof["avg_us"] = dom["avg_us"]
    roof["units_per_launch"] = dom["flops"] if roof["unit"] == "TFLOP/s" else dom["bytes"]

    dtypes = sorted({wl.dtype for _, wl, _, _ in preps})
    config = {"workload": a.workload, "calls": [wl.name for _, wl, _, _ in preps], "dtypes": dtypes,
              "rotation_sets": R,
              "timing": ("wall clock over K steps" + (" (one HIP graph replay per step)" if a.graph else
                                                      " (eager launches)") +
                         "; per-call HIP events on the launch stream around eager launches"),
              "schedules": "planner rule" if a.rule else "timed at plan time (conv_tune), fastest kept",
              "headline": ("sum over the calls of their time at the roofline / measured step time"
                           if a.workload in META else "algorithmic units of a step / measured step time")}
    out = {"metric": METRIC, "value": round(value, 3), "unit": unit, "n_gpus": 1, "steps": a.steps,
           "warmup": a.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": dtypes[0] if len(dtypes) == 1 else "mixed",
           "data": "synthetic", "config": config, "roofline": roof, "per_workload": rows, "per_call": per_call}
    if a.no_cpu_baseline:
        out["cpu_baseline"] = None
    else:
        out["cpu_baseline"] = cpu_baseline(calls, a.cpu_seconds, value if a.workload in META else None)
        if a.workload not in META:
            # Single-workload runs: the CPU figure in the workload's own unit.
            pw = out["cpu_baseline"]["per_workload"][0]
            out["cpu_baseline"].update(value=pw["value"], unit=pw["unit"])
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
