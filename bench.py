#!/usr/bin/env python3
"""Benchmark of the fused linear layer out = act(A@B + bias) on one MI355X.

One step = one fused_linear call (bias, activation, cast and store fused into
the GEMM) over the workload's synthetic inputs, already resident in HBM.
Prints ONE JSON line with the throughput (TFLOP/s = 2*M*N*K / step time),
the roofline of the fused kernel (measured with HIP events on the stream the
kernels run on), the unfused three-kernel chain for comparison, and the
FP64 CPU oracle timed on a bounded sample of the same workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                       [--prewarm-s S] [--no-cpu-baseline] [--no-unfused]
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fused GEMM+bias+act TFLOP/s and % of MFMA peak (fp16, 4096^3) on 1 MI355X"
DEFAULT_WORKLOAD = "relu_f16_4096x4096x4096"
# MI355X dense matrix peaks (TFLOP/s) and HBM bandwidth (GB/s): 256 CUs at
# 2.4 GHz; fp16/bf16 4096 flop/clk/CU, fp32 256 flop/clk/CU.
PEAK_TFLOPS = {"f16": 2516.6, "bf16": 2516.6, "f32": 157.3, "fp8": 5033.2}
PEAK_HBM_GBS = 8000.0
MALL_BYTES = 256 << 20      # MI355X last-level cache (Infinity Cache) in front of HBM
MALL_NOTE = ("the passes' (M,N) arrays fit in the 256 MB MALL and stay there between passes, so their GB/s "
             "can exceed the HBM peak (frac_hbm > 1)")
ES = {"f32": 4, "f16": 2, "bf16": 2}


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=100)
    p.add_argument("--warmup", type=int, default=50)
    p.add_argument("--prewarm-s", type=float, default=0.5,
                   help="seconds of untimed steps before the warm-up steps (lets the GPU reach its sustained clock)")
    p.add_argument("--workload", default=DEFAULT_WORKLOAD)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-unfused", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU-oracle sample time")
    p.add_argument("--group-m", type=int, default=0)
    p.add_argument("--persistent", type=int, default=0)
    p.add_argument("--tile-cfg", type=int, default=0, help="fl_options.tile_cfg (0 = automatic)")
    p.add_argument("--shape", default="",
                   help="MxNxK: the workload's kind and data recipe at another size (a study, not a bench line "
                        "of the named workload)")
    p.add_argument("--calib-copy-mib", type=int, default=0,
                   help="also run a plain device copy of this many MiB (counter calibration)")
    return p.parse_args()


def source_hash(files=None):
    """Hash of the kernel sources (all of csrc/, or the listed files) with
    comments and whitespace removed, so that counters recorded for a kernel
    stay valid across comment edits and become stale on any change to the
    code it is built from."""
    import re
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "activation_epilogue_amd", "csrc")
    for name in sorted(files or os.listdir(csrc)):
        with open(os.path.join(csrc, name), encoding="utf-8") as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(name.encode() + " ".join(text.split()).encode())
    return h.hexdigest()[:16]


def measured_traffic(workload):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the kernel source as it is now; else None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path))
    except ValueError:
        return None
    if rec.get("source_hash") != source_hash(rec.get("sources")):
        return None
    return rec.get("bytes_per_launch")


def time_loop(fn, steps, warmup, stream):
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record(stream)
    for _ in range(steps):
        fn()
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return start.elapsed_time(end) / steps, wall / steps * 1e3


def launch_times(fn, n, stream, scrub=None):
    """Per-launch durations (ms) of n calls, each bracketed by its own HIP
    events on the kernel's stream, after the timed region.  With scrub (a
    device buffer), the buffer is overwritten before every call, so the
    operands no longer sit in the L2 or the 256 MB MALL (a cold call)."""
    import torch
    evs = []
    for _ in range(n):
        if scrub is not None:
            scrub.fill_(1)
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record(stream)
        fn()
        e.record(stream)
        evs.append((s, e))
    torch.cuda.synchronize()
    ts = sorted(s.elapsed_time(e) for s, e in evs)
    return {"n": n, "median_ms": round(ts[n // 2], 4), "min_ms": round(ts[0], 4), "max_ms": round(ts[-1], 4)}


def algorithmic_bytes(M, N, K, es, act, residual=False, qfmt=None, in8=False, bwd=False):
    """Bytes one launch must move at least: each input read once and each
    output written once.  Forward: A (M,K) and B (K,N) (one byte per element
    for FP8 operands), bias (N,), Y (gate) and R (residual) (M,N), and out
    (M,N) in the I/O dtype, or one byte per element for a quantized output.
    Backward epilogue: G (M,K), W (N,K), the saved X (M,N) (+ Y) read, dX (+
    dY) written, and the fp32 bias gradient (N,) zeroed and added to."""
    glu = act == "glu"
    if bwd:
        return (M * K + K * N + 2 * M * N * (2 if glu else 1)) * es + 2 * N * 4
    mn_arrays = (0 if qfmt else 1) + glu + bool(residual)  # out, Y, R in the I/O dtype
    return ((M * K + K * N) * (1 if in8 else es) + (N + M * N * mn_arrays) * es + (M * N if qfmt else 0))


def activation_traffic_bytes(M, N, es, act, kernels=3):
    """HBM bytes of the (M,N) activation arrays around the product ("Triton:
    Fused Matmul + Bias + ReLU (Epilogue Fusion)", "The HBM traffic";
    "Optimizing GEMM + Activation on CDNA4 with TLX", "The GLU Block").
    Fused: the output written once, plus Y read by the gate.  Unfused, three
    kernels (this library's chain): the product stores X; the bias pass reads
    and writes it; the activation pass reads it (and Y) and writes the
    output.  Unfused, two kernels (the bias folded into the product, as a
    library GEMM does): X written, X (and Y) read, the output written."""
    glu = 1 if act == "glu" else 0
    mn = M * N * es
    if kernels == 3:
        unfused = (5 + glu) * mn
    elif kernels == 2:
        unfused = (3 + glu) * mn
    else:
        raise ValueError("kernels is 2 or 3")
    return {"fused": (1 + glu) * mn, "unfused": unfused}


# The TLX page's own table ("Optimizing GEMM + Activation on CDNA4 with
# TLX", the benchmark after Version 4): its best fused gate kernel on one
# MI350X, fp16, M=1024, N=21568, TFLOP/s by K.  Another machine: context
# for the same workloads, not a target.
PAGES_GATE_MI350X = {256: 357.0, 512: 502.0, 1024: 619.0}


def device_info():
    import torch
    p = torch.cuda.get_device_properties(0)
    return {"name": p.name, "arch": getattr(p, "gcnArchName", None), "cus": p.multi_processor_count}


def cpu_model():
    """The host CPU as /proc/cpuinfo names it, with its family / model /
    stepping numbers and the logical CPUs visible to this process."""
    info = {}
    try:
        for line in open("/proc/cpuinfo"):
            k, _, v = line.partition(":")
            k = k.strip()
            if k in ("model name", "cpu family", "model", "stepping") and k not in info:
                info[k] = v.strip()
    except OSError:
        pass
    info["logical_cpus"] = os.cpu_count()
    try:
        info["usable_cpus"] = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        pass
    return info


def _oracle_rows(w, d, rows, threads=None):
    """The oracle's output for the given rows of the workload (FP64 inside,
    rounded once to the output type), as its own storage arrays."""
    import oracle
    if w.bwd:
        return oracle.fused_linear_bwd(d["G"], d["W"], d["X"], d["Y"], act=w.act, dtype=w.dtype, rows=rows,
                                       threads=threads)
    if w.in8:
        return oracle.fused_linear_fp8(d["A8"], d["B8"], d["ab_scale"], d["bias"], d["Y"], act=w.act,
                                       out_dtype=w.dtype, rows=rows, threads=threads)
    if w.qfmt:
        return oracle.fused_linear_quant(d["A"], d["B"], d["bias"], d["Y"], act=w.act, dtype=w.dtype, qfmt=w.qfmt,
                                         scale=w.scale, rows=rows, threads=threads, want_u=True)
    return oracle.fused_linear(d["A"], d["B"], d["bias"], d["Y"], act=w.act, dtype=w.dtype, rows=rows, R=d["R"],
                               threads=threads)


def cpu_baseline(w, d, target_s):
    """Time the FP64 oracle (as it is) on a bounded sample of output rows,
    growing the sample until one call takes at least half of target_s.
    Returns the baseline record and the rows and oracle output of the sample
    (for the parity statistics)."""
    import numpy as np
    import oracle
    threads = oracle.max_threads()
    nrows = min(threads, w.M)
    while True:
        rows = np.linspace(0, w.M - 1, nrows).astype(np.int64)
        t0 = time.perf_counter()
        ref = _oracle_rows(w, d, rows)
        dt = time.perf_counter() - t0
        if dt >= 0.5 * target_s or nrows >= w.M:
            break
        nrows = int(min(w.M, nrows * max(2.0, min(16.0, target_s / max(dt, 1e-3)))))
    flops = 2.0 * nrows * w.N * w.K
    rec = {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
           "cpu": cpu_model(),
           "sample": f"{nrows} of {w.M} output rows of {w.name}, FP64, evenly spaced; "
                     f"{flops / 2:.3g} multiply-adds in {dt:.1f} s (B decoded once per call)"}
    return rec, rows, ref


def per_core_rate():
    """The oracle on one thread: the whole 127x129x96 fp32 ReLU workload
    (repeated for at least 0.5 s) and 16 evenly spaced rows of the ragged
    4097x3071x1537 bf16 one, in GFLOP/s of the GEMM (2*M*N*K)."""
    import numpy as np
    import oracle
    from activation_epilogue_amd import synth
    out = {}
    for name, nrows in (("relu_f32_127x129x96", None), ("relu_bf16_4097x3071x1537", 16)):
        w = synth.WORKLOADS[name]
        d = synth.draw_workload(w)
        rows = None if nrows is None else np.linspace(0, w.M - 1, nrows).astype(np.int64)
        n_out = w.M if rows is None else nrows
        reps, t0 = 0, time.perf_counter()
        while True:
            oracle.fused_linear(d["A"], d["B"], d["bias"], d["Y"], act=w.act, dtype=w.dtype, rows=rows, threads=1)
            reps += 1
            dt = time.perf_counter() - t0
            if dt >= 0.5:
                break
        out[name] = {"GFLOP/s": round(2.0 * n_out * w.N * w.K * reps / dt / 1e9, 3), "threads": 1,
                     "rows": "all" if rows is None else f"{nrows} of {w.M}", "calls": reps}
    return out


def parity_stats(w, host_out, ref):
    """Element-wise comparison of the benchmarked output rows with the
    oracle's: max |dev - ref|, max relative error and the number of elements
    outside the stated tolerance (or, for one-byte codes, outside the
    boundary band)."""
    import oracle
    if w.qfmt:
        codes, u = ref
        r = oracle.compare_quant(host_out, codes, u, w.qfmt)
        return {"elements": int(host_out.size), "violations": r["mismatches"],
                "accepted_near_boundary": r["accepted_near_boundary"], "ok": bool(r["ok"]),
                "tolerance": "code equal, or neighbouring code within the binary32 boundary band"}
    if w.bwd:
        ref = ref[0]  # dX
    atol, rtol = oracle.TOLERANCE[w.dtype]
    r = oracle.compare(host_out, ref, w.dtype)
    return {"elements": int(host_out.size), "max_abs": r["max_abs"], "max_rel": r["max_rel"],
            "violations": r["violations"], "ok": r["ok"], "tolerance": {"atol": atol, "rtol": rtol}}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build runs on a single MI355X and has no multi-GPU "
              "path (the layer shards by output columns or rows with no communication; see DESIGN.md).",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import activation_epilogue_amd as fl
    from activation_epilogue_amd import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    fl.load_library()
    w = synth.WORKLOADS[args.workload]
    if args.shape:
        M, N, K = (int(x) for x in args.shape.split("x"))
        w = dataclasses.replace(w, name=f"{w.name}@{M}x{N}x{K}", M=M, N=N, K=K)
    tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[w.dtype]
    d = synth.draw_workload(w)

    def dev(raw):
        if raw is None:
            return None
        t = torch.from_numpy(np.ascontiguousarray(raw))
        if w.dtype == "bf16":
            t = t.view(torch.int16).view(torch.bfloat16)
        return t.to("cuda")

    if w.in8:
        A, B = (torch.from_numpy(d[k]).to("cuda") for k in ("A8", "B8"))
    elif w.bwd:
        # the backward epilogue: A = G (M,K), B = W (N,K), saved X, gate Y
        A, B, Xs = dev(d["G"]), dev(d["W"]), dev(d["X"])
        dY = torch.empty((w.M, w.N), dtype=tdt, device="cuda") if w.act == "glu" else None
        dbias = torch.empty((w.N,), dtype=torch.float32, device="cuda")
    else:
        A, B = dev(d["A"]), dev(d["B"])
    bias, Y, R = dev(d.get("bias")), dev(d["Y"]), dev(d.get("R"))
    out = torch.empty((w.M, w.N), dtype=torch.uint8 if w.qfmt else tdt, device="cuda")
    stream = torch.cuda.current_stream()
    opts = {}
    if args.group_m:
        opts["group_m"] = args.group_m
    if args.persistent:
        opts["persistent"] = 1
    if args.tile_cfg:
        opts["tile_cfg"] = args.tile_cfg
    code = {"f32": 0, "f16": 1, "bf16": 2}[w.dtype]
    bm, bn, tiles_m, tiles_n = fl.tile_grid(w.M, w.N, w.K, code, **opts)
    if w.bwd and not args.tile_cfg and bn != 256:
        # the backward entry point runs 256x128 where the automatic choice
        # names the two-per-CU or the 256x192 kernel (not built there)
        bm, bn, tiles_m, tiles_n = fl.tile_grid(w.M, w.N, w.K, code, **dict(opts, tile_cfg=2))
    kernel = ("fused_linear_bwd_kernel" if w.bwd else
              "fused_linear_kernel" if (w.dtype == "f32" or args.tile_cfg == 3) else "fused_linear_dma16_kernel")

    def step():
        if w.bwd:
            fl.fused_linear_bwd(A, B, Xs, Y, act=w.act, dX=out, dY=dY, dbias=dbias, **opts)
        elif w.in8:
            fl.fused_linear_fp8(A, B, d["ab_scale"], bias, Y, act=w.act, out_dtype=tdt, out=out, **opts)
        elif w.qfmt:
            fl.fused_linear_quant(A, B, bias, Y, act=w.act, scale=w.scale, qfmt=w.qfmt, out=out, **opts)
        else:
            fl.fused_linear(A, B, bias, Y, act=w.act, out=out, R=R, **opts)

    # The shader clock ramps up over the first ~100 ms of load; time the
    # sustained state.  These untimed steps precede the W warm-up steps.
    t_end = time.perf_counter() + args.prewarm_s
    while time.perf_counter() < t_end:
        for _ in range(20):
            step()
        torch.cuda.synchronize()
    ms_event, ms_wall = time_loop(step, args.steps, args.warmup, stream)
    # Outside the timed region: per-launch durations (median / min), warm and
    # with a 512 MiB scrub buffer written before each call (cold caches).
    warm = launch_times(step, 20, stream)
    scrub = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    cold = launch_times(step, 20, stream, scrub=scrub)
    del scrub
    if args.calib_copy_mib:
        # A plain copy of known size, outside the timed region, so that memory
        # counters taken over this run can be scaled to bytes.
        src = torch.empty(args.calib_copy_mib << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    flops = w.flops
    tflops = flops / (ms_wall * 1e-3) / 1e12
    achieved = flops / (ms_event * 1e-3) / 1e12
    peak = PEAK_TFLOPS["fp8" if w.in8 else w.dtype]
    es = ES[w.dtype]
    alg_bytes = algorithmic_bytes(w.M, w.N, w.K, es, w.act, residual=w.residual, qfmt=w.qfmt, in8=w.in8, bwd=w.bwd)

    result = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "prewarm_s": args.prewarm_s,
        "ms_per_step": round(ms_wall, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8->" + w.dtype if w.in8 else w.dtype,
        "data": ("synthetic (seeded numpy PCG64: G ~ N(0,1), W ~ N(0,1/K), X ~ N(0,1)%s)" % (
            ", Y ~ U(-1,1)" if w.act == "glu" else "") if w.bwd else
            "synthetic (seeded numpy PCG64: %s, bias ~ N(0,%g)%s%s)" % (
            "A,B ~ N(0,1) as FP8 E4M3 codes, ab_scale 1/sqrt(K)" if w.in8 else "A,B ~ N(0,1/K)",
            w.bias_var, ", Y ~ U(-1,1)" if w.act == "glu" else "", ", R ~ N(0,1)" if w.residual else "")),
        "config": {"workload": w.name, "M": w.M, "N": w.N, "K": w.K, "act": w.act, "residual": w.residual,
                   "out": w.qfmt or w.dtype, "scale": w.scale if w.qfmt else None,
                   "operands": "fp8_e4m3" if w.in8 else w.dtype,
                   "pass": "backward: dX = (G @ W^T) * act'(X), dbias" if w.bwd else "forward",
                   "io_dtype": w.dtype,
                   "accumulate": "f32", "tile": f"{bm}x{bn}", "tiles": tiles_m * tiles_n,
                   "tile_cfg": args.tile_cfg, "group_m": args.group_m or 4, "persistent": bool(args.persistent)},
        "frac_of_peak": round(tflops / peak, 4),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(achieved / peak, 4), "traffic": measured_traffic(w.name),
                     "kernel": kernel, "avg_launch_ms": round(ms_event, 4),
                     "algorithmic_bytes": alg_bytes},
        "launches": {"warm": warm, "cold_512MiB_scrub": cold,
                     "cold_tflops_median": round(flops / (cold["median_ms"] * 1e-3) / 1e12, 2)},
        "device": device_info(),
    }

    if w.bwd and not args.no_unfused:
        # the unfused backward chain: the product stored, an elementwise
        # derivative pass, a column-sum pass (each one launch, storing its result)
        Dbuf = torch.empty_like(out)
        dXu = torch.empty_like(out)
        dYu = torch.empty_like(out) if w.act == "glu" else None
        dbu = torch.empty_like(dbias)

        def chain():
            fl.gemm_nt(A, B, Dbuf)
            fl.activation_grad(Dbuf, Xs, Y, act=w.act, dX=dXu, dY=dYu)
            fl.column_sum(dXu, dbu)

        ms_chain, _ = time_loop(chain, args.steps, args.warmup, stream)
        ms_gemm, _ = time_loop(lambda: fl.gemm_nt(A, B, Dbuf), args.steps, args.warmup, stream)
        ms_ag, _ = time_loop(lambda: fl.activation_grad(Dbuf, Xs, Y, act=w.act, dX=dXu, dY=dYu), args.steps,
                             args.warmup, stream)
        ms_cs, _ = time_loop(lambda: fl.column_sum(dXu, dbu), args.steps, args.warmup, stream)
        mn = w.M * w.N
        glu = w.act == "glu"
        ag_bytes = (3 + 2 * glu) * mn * es  # D, X (+Y) read, dX (+dY) written
        cs_bytes = mn * es + w.N * 4
        result["unfused"] = {
            "ms_per_step": round(ms_chain, 4),
            "fused_speedup": round(ms_chain / ms_event, 3),
            "gemm_nt_ms": round(ms_gemm, 4),
            "activation_grad_pass": {"ms": round(ms_ag, 4), "GB/s": round(ag_bytes / ms_ag / 1e6, 1),
                                     "frac_hbm": round(ag_bytes / ms_ag / 1e6 / PEAK_HBM_GBS, 3)},
            "column_sum_pass": {"ms": round(ms_cs, 4), "GB/s": round(cs_bytes / ms_cs / 1e6, 1),
                                "frac_hbm": round(cs_bytes / ms_cs / 1e6 / PEAK_HBM_GBS, 3)},
            # bytes of the (M,N) arrays beyond the product's own operands: fused reads X (+Y) and
            # writes dX (+dY); the chain also writes and re-reads D and re-reads dX
            "epilogue_traffic_bytes": {"fused": (2 + 2 * glu) * mn * es, "unfused": (5 + 2 * glu) * mn * es},
        }
        if ag_bytes <= MALL_BYTES:
            result["unfused"]["note"] = MALL_NOTE
    elif w.residual or w.qfmt or w.in8 or w.bwd:
        result["unfused"] = None  # the unfused chain has no residual, quantizing or FP8 form
    elif not args.no_unfused:
        X = torch.empty_like(out)

        def chain():
            fl.gemm(A, B, X)
            fl.bias_add(X, bias)
            fl.activation(X, Y, out=X, act=w.act)

        ms_chain, _ = time_loop(chain, args.steps, args.warmup, stream)
        ms_gemm, _ = time_loop(lambda: fl.gemm(A, B, X), args.steps, args.warmup, stream)
        ms_bias, _ = time_loop(lambda: fl.bias_add(X, bias), args.steps, args.warmup, stream)
        ms_act, _ = time_loop(lambda: fl.activation(X, Y, out=X, act=w.act), args.steps, args.warmup, stream)
        mn = w.M * w.N
        bias_bytes = (2 * mn + w.N) * es
        act_bytes = (3 if w.act == "glu" else 2) * mn * es
        result["unfused"] = {
            "ms_per_step": round(ms_chain, 4),
            "fused_speedup": round(ms_chain / ms_event, 3),
            "gemm_ms": round(ms_gemm, 4),
            "bias_pass": {"ms": round(ms_bias, 4), "GB/s": round(bias_bytes / ms_bias / 1e6, 1),
                          "frac_hbm": round(bias_bytes / ms_bias / 1e6 / PEAK_HBM_GBS, 3)},
            "act_pass": {"ms": round(ms_act, 4), "GB/s": round(act_bytes / ms_act / 1e6, 1),
                         "frac_hbm": round(act_bytes / ms_act / 1e6 / PEAK_HBM_GBS, 3)},
            "activation_traffic_bytes": activation_traffic_bytes(w.M, w.N, es, w.act),
            "activation_traffic_bytes_two_kernels": activation_traffic_bytes(w.M, w.N, es, w.act, kernels=2),
        }
        if act_bytes <= MALL_BYTES:
            result["unfused"]["note"] = MALL_NOTE

    if (w.act == "glu" and not w.bwd and not w.in8 and not w.residual and w.dtype == "f16"
            and (w.M, w.N) == (1024, 21568) and w.K in PAGES_GATE_MI350X):
        ref = PAGES_GATE_MI350X[w.K]
        result["pages_context"] = {"value": ref, "unit": "TFLOP/s", "hardware": "1x MI350X",
                                   "kernel": "the TLX page's Version 4", "ratio": round(tflops / ref, 3)}
    if not args.no_cpu_baseline:
        import numpy as np
        result["cpu_baseline"], rows, ref = cpu_baseline(w, d, args.cpu_seconds)
        result["cpu_baseline"]["per_core"] = per_core_rate()
        # the output the timed steps wrote, on the sampled rows, against the oracle
        step()
        torch.cuda.synchronize()
        host = out.detach().to("cpu")
        if w.qfmt:
            host = host.numpy()
        elif w.dtype == "bf16":
            host = host.view(torch.int16).numpy().view(np.uint16)
        else:
            host = host.numpy()
        result["parity"] = dict(parity_stats(w, np.ascontiguousarray(host[rows]), ref),
                                rows=f"{len(rows)} of {w.M} (the CPU baseline's sample)")

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
