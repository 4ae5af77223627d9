#!/usr/bin/env python3
"""Benchmark of the inline-quantized A4W4 MXFP4 GEMM on one MI355X.

Headline workload (one "step"): the dense GEMM N=8448, K=7168, the largest weight of the
microbenchmark sweep, at every M of it (1, 8, 32, 128, 512, 2048), one call per M, each with
bf16 activations quantized by the library (inside the kernel, or once into the workspace at
large M) against a prepared MXFP4 weight; weight preparation is outside the timed region, as
in "[gfx950][FlyDSL] Add direct dense A4W4 MXFP4 GEMM", Kernel microbenchmark. Inputs are
synthetic (seeded, see workloads/).

Timing: every timed region is HIP graph replays bracketed by HIP events on the stream the
graphs are launched on. Buffers rotate over R distinct (A, prepared W, C) sets so the working
set exceeds the 256 MB Infinity Cache ("cold"); single-set ("warm") times are reported as
context. The step is one graph replay per step, each timed: the value is the median step,
with the spread. Per-point times are the median over 5 replays of a graph of many launches.

Output: one JSON line (rank 0, N=1) with the headline step, the roofline of the dominant
call, the CPU oracle baseline, and the full sweep (all dense points with their relative L2
against the unquantized bf16 product, the A16WFP4 variant, and the MoE layer's grouped
GEMMs) under "sweep".
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "A4W4 GEMM us + %HBM roofline (M<=32) / %MXFP4 MFMA peak (M>=512)"
HBM_PEAK = 8.0e12            # B/s, MI355X HBM3E
MFMA_FP4_PEAK = 10.1e15      # flop/s, MI355X dense MXFP4
MFMA_BF16_PEAK = 2.5e15      # flop/s, MI355X dense bf16 (the A16WFP4 variant's MFMA)
MALL_BYTES = 256 << 20       # Infinity Cache
ROTATE_TARGET = 1 << 30      # bytes touched per rotation cycle (4x the Infinity Cache)
HEADLINE = "n8448_k7168"
REPLAYS = 5                  # graph replays per sweep point (median and spread)
# The pages' direct-kernel median times ("[gfx950][FlyDSL] Add direct dense A4W4 MXFP4 GEMM",
# Kernel microbenchmark table); the headline compares against their sum over its M sweep.
PAGE_US = {("n7168_k768", 1): 12.580, ("n7168_k768", 8): 11.921, ("n7168_k768", 32): 12.120,
           ("n7168_k768", 128): 12.380, ("n7168_k768", 512): 15.520, ("n7168_k768", 2048): 31.700,
           ("n7168_k4224", 1): 15.960, ("n7168_k4224", 8): 23.041, ("n7168_k4224", 32): 23.520,
           ("n7168_k4224", 128): 23.280, ("n7168_k4224", 512): 50.041, ("n7168_k4224", 2048): 107.041,
           ("n1536_k7168", 1): 18.420, ("n1536_k7168", 8): 23.320, ("n1536_k7168", 32): 26.181,
           ("n1536_k7168", 128): 28.300, ("n1536_k7168", 512): 29.621, ("n1536_k7168", 2048): 65.081,
           ("n8448_k7168", 1): 23.201, ("n8448_k7168", 8): 26.940, ("n8448_k7168", 32): 30.240,
           ("n8448_k7168", 128): 60.121, ("n8448_k7168", 512): 89.480, ("n8448_k7168", 2048): 237.863}


def algo_bytes(M, N, K):
    """Prepared MXFP4 weight (N*K*17/32) + bf16 activations + bf16 output."""
    return N * K * 17 // 32 + 2 * M * K + 2 * M * N


def algo_flops(M, N, K):
    return 2 * M * N * K


def log(msg):
    print(msg, file=sys.stderr, flush=True)


# ----------------------------------------------------------------------------- GPU timing

class Timer:
    def __init__(self, torch):
        self.torch = torch

    def graph(self, launches):
        """Capture the callables (each enqueues kernels on the current stream) in one graph."""
        torch = self.torch
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            launches[0]()
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for f in launches:
                f()
        torch.cuda.synchronize()
        return g

    def replay_ms(self, g, reps=1):
        torch = self.torch
        g.replay()
        torch.cuda.synchronize()
        st = torch.cuda.current_stream()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(st)
        for _ in range(reps):
            g.replay()
        e1.record(st)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps


def dev_bf16(torch, bits):
    import numpy as np
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16).copy()).view(torch.bfloat16).cuda()


class DensePoint:
    """R rotating buffer sets for one (N, K, M) point."""

    def __init__(self, torch, mx, wp, a_bits, N, K, M, rotate=True):
        self.N, self.K, self.M = N, K, M
        per = wp.numel() + 2 * M * K + 2 * M * N
        self.R = max(1, min(256, math.ceil(ROTATE_TARGET / per))) if rotate else 1
        a = dev_bf16(torch, a_bits)
        self.sets = []
        for r in range(self.R):
            w_r = wp if r == 0 else wp.clone()
            a_r = a if r == 0 else a.clone()
            c_r = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
            self.sets.append((a_r, w_r, c_r))
        self.mx = mx

    def launch(self, i):
        a, w, c = self.sets[i % self.R]
        return lambda: self.mx.mx_a4w4_gemm(a, w, self.N, out=c)


def replay_stats(timer, g, launches, replays=REPLAYS):
    """(median, min, max) microseconds per launch over `replays` timed replays of g."""
    per = sorted(timer.replay_ms(g, reps=1) * 1e3 / launches for _ in range(replays))
    return per[len(per) // 2], per[0], per[-1]


def time_point(timer, pt, launches=200):
    g = timer.graph([pt.launch(i) for i in range(launches)])
    st = replay_stats(timer, g, launches)
    del g
    return st


def calibrate(torch, mx, timer):
    """Measured ceilings on this device: a plain streaming read of 1 GiB (4x the Infinity
    Cache, so it comes from HBM) and an MFMA-only FP4 loop; best of a few launch shapes."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    buf = torch.zeros(1 << 30, dtype=torch.uint8, device="cuda")
    read = []
    for per_cu in (2, 4, 8):
        g = timer.graph([lambda c=cus * per_cu: mx.mx_calib_read(buf, c, sink)] * 10)
        ms = timer.replay_ms(g, reps=2) / 10
        del g
        read.append((buf.numel() / ms / 1e6, per_cu))
    del buf
    torch.cuda.empty_cache()
    # the floor for streaming the largest prepared weight once: a cold 32 MiB read, rotating
    # over 32 buffers (1 GiB) so each read comes from HBM, best launch shape
    small = [torch.zeros(32 << 20, dtype=torch.uint8, device="cuda") for _ in range(32)]
    read32 = []
    for ctas in (cus * 2, cus * 8):
        g = timer.graph([lambda b=small[i % 32], c=ctas: mx.mx_calib_read(b, c, sink) for i in range(64)])
        read32.append(replay_stats(timer, g, 64)[0])
        del g
    del small
    torch.cuda.empty_cache()
    mfma = []
    iters = 2048
    for per_cu in (2, 4):
        ctas = cus * per_cu
        g = timer.graph([lambda c=ctas: mx.mx_calib_mfma(c, iters, sink)] * 5)
        ms = timer.replay_ms(g, reps=2) / 5
        del g
        mfma.append((mx.mx_calib_mfma_flops(ctas, iters) / ms / 1e9, per_cu))
    best_r, best_m = max(read), max(mfma)
    return {"hbm_read_GBps": round(best_r[0], 1), "mfma_fp4_TFLOPs": round(best_m[0], 1),
            "read_32mb_us": round(min(read32), 3),
            "read_32mb": "cold 32 MiB streaming read (rotating over 1 GiB), median of 5 replays of 64 reads, "
                         "best of 2 and 8 CTAs per CU: the floor for streaming the 8448 x 7168 weight once",
            "read": "1 GiB streaming read, 16-byte coalesced loads, %d CTAs of 256 threads per CU" % best_r[1],
            "mfma": "16x16x128 block-scaled FP4 MFMA on registers, 8 chains per wave, %d CTAs of 4 waves "
                    "per CU" % best_m[1],
            "cus": cus}


def calibrate_mfma_data(torch, mx, timer, ops, cus):
    """The FP4 MFMA rate on the GEMM's own operand bits (the bytes of a prepared weight):
    one wave per SIMD, 64 accumulators, the block products a 128 x 128 wave tile issues per
    K step. The device holds a lower clock under random-looking operands than under the
    fixed ones of the plain MFMA loop, so this is the ceiling a GEMM on this data can reach."""
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    iters = 1024
    rates = []
    for _ in range(2):
        g = timer.graph([lambda: mx.mx_calib_mfma_operands(ops, cus, iters, sink)] * 4)
        ms = timer.replay_ms(g, reps=2) / 4
        del g
        rates.append(mx.mx_calib_mfma_operands_flops(cus, iters) / ms / 1e9)
    return round(max(rates), 1)


def calibrate_mfma_clock(torch, mx, ops, cus):
    """The shader clock and the cycles per MFMA during the same loop, on the weight's own
    operand bytes and on constant bytes (every E2M1 code 1.0): each wave's core-clock ticks
    over its loop against the 100 MHz counter. It runs right after the rate calibration on
    the same loop; of four launches per operand set the last one's waves are read, and the
    median wave is reported."""
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    clocks = torch.zeros(8 * cus, dtype=torch.int64, device="cuda")
    const = torch.full((16384,), 0x22, dtype=torch.uint8, device="cuda")
    iters, out = 4096, {}
    for name, src in (("data", ops), ("constant", const)):
        for _ in range(4):
            mx.mx_calib_mfma_operands_clock(src, cus, iters, sink, clocks)
        torch.cuda.synchronize()
        c = clocks.view(-1, 2).double().cpu()
        ghz = (c[:, 0] / (c[:, 1] / 100e6) / 1e9).median().item()
        cyc = (c[:, 0] / (iters * 64)).median().item()
        out[f"mfma_clock_GHz_{name}"] = round(ghz, 3)
        out[f"mfma_cycles_per_op_{name}"] = round(cyc, 2)
    return out


def point_record(name, N, K, M, cold, us_warm, kernel=None):
    """cold: (median, min, max) us per launch over the replays."""
    us_cold = cold[0]
    B, F = algo_bytes(M, N, K), algo_flops(M, N, K)
    t_hbm, t_mfma = B / HBM_PEAK * 1e6, F / MFMA_FP4_PEAK * 1e6
    rec = {
        "workload": name, "N": N, "K": K, "M": M,
        "us": round(us_cold, 3), "us_min": round(cold[1], 3), "us_max": round(cold[2], 3),
        "us_warm": round(us_warm, 3),
        "tflops": round(F / us_cold / 1e6, 2), "gbps": round(B / us_cold / 1e3, 1),
        "frac_hbm": round(t_hbm / us_cold, 4), "frac_mfma": round(t_mfma / us_cold, 4),
        "binds": "hbm" if t_hbm >= t_mfma else "mfma",
        "frac_binding": round(max(t_hbm, t_mfma) / us_cold, 4),
    }
    if (name, M) in PAGE_US:
        rec["page_us"] = PAGE_US[(name, M)]
    if kernel:
        rec["kernel"] = kernel
    return rec


def kernel_name(mx, M, N, K):
    """The kernel instantiation(s) the library launches for this shape when handed the
    workspace it asks for (what the binding does by default)."""
    return mx.mx_a4w4_gemm_plan(M, N, K, mx.mx_a4w4_gemm_workspace_bytes(M, N, K))


# ----------------------------------------------------------------------------- HBM traffic

TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
KERNEL_SOURCES = ["mxfp4_quantized_gemm_inline_amd/csrc/mx_kernels.hip",
                  "mxfp4_quantized_gemm_inline_amd/csrc/mx_gemm_qo.hip",
                  "mxfp4_quantized_gemm_inline_amd/csrc/mx_device.h"]


LAUNCHERS_MARK = b"// ====================================================================== launchers"


def kernel_source_hash():
    """Hash of the device code: mx_device.h, and mx_kernels.hip and mx_gemm_qo.hip up to their
    host launchers (configuration selection there does not change a kernel)."""
    import hashlib
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            src = f.read()
        cut = src.find(LAUNCHERS_MARK)
        h.update(src if cut < 0 else src[:cut])
    return h.hexdigest()[:16]


def recorded_traffic(kernel, workload, M):
    """Calibrated HBM bytes per launch from the committed counter summary, or None when there
    is none for this kernel and point or the kernel sources changed since it was taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            recs = json.load(f)
    except (OSError, ValueError):
        return None
    for r in recs:
        if r.get("kernel") == kernel and r.get("workload") == workload and r.get("M") == M:
            if r.get("source_hash") != kernel_source_hash():
                return None
            return int(r["traffic_bytes"])
    return None


def _counter_rows(d):
    """(kernel name, counter, value) rows from every rocprofv3 counter CSV under d."""
    import csv
    rows = []
    for root, _, files in os.walk(d):
        for fn in files:
            if fn.endswith("counter_collection.csv"):
                with open(os.path.join(root, fn)) as f:
                    for r in csv.DictReader(f):
                        rows.append((r["Kernel_Name"], r["Counter_Name"], float(r["Counter_Value"])))
    return rows


def plan_kernels(plan):
    """The kernels of a plan string, e.g. "k_prepare + k_gemm_qo<2, 2, 4, 4, 4, 2> GM=8" gives
    ["k_prepare", "k_gemm_qo<2, 2, 4, 4, 4, 2>"]."""
    import re
    return [m.group(0) for m in re.finditer(r"\bk_\w+(<[^>]*>)?", plan)]


def dispatch_matches(kernel, name):
    """True when a profiler kernel name is a dispatch of `kernel` (template arguments included;
    a plain name must be followed by its argument or template list, so k_prepare is not
    k_prepare_packed)."""
    if "<" in kernel:
        return kernel in name
    return (kernel + "(") in name or (kernel + "<") in name


def summarize_counters(fetch_dir, write_dir, workload, M, copy_mib):
    """FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of every kernel of the GEMM call's plan, each
    scaled by the factor that maps the same counter on a plain copy of copy_mib MiB to its true
    size, summed over the plan's kernels (bytes per call)."""
    import mxfp4_quantized_gemm_inline_amd as mx
    import workloads as W
    N, K = W.DENSE_CONFIGS[workload][:2]
    plan = mx.mx_a4w4_gemm_plan(M, N, K, mx.mx_a4w4_gemm_workspace_bytes(M, N, K))
    kernels = plan_kernels(plan)
    out = {"kernel": plan, "workload": workload, "N": N, "K": K, "M": M, "copy_mib": copy_mib, "per_kernel": {}}
    total = 0.0
    for ctr, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = [r for r in _counter_rows(d) if r[1] == ctr]
        copy = [v for n, c, v in rows if "copybuffer" in n.lower()]
        if not copy:
            raise SystemExit(f"{ctr}: no copy dispatch under {d}")
        factor = copy_mib * 1024.0 / max(copy)
        out[ctr.lower() + "_factor"] = round(factor, 4)
        for k in kernels:
            vals = [v for n, c, v in rows if dispatch_matches(k, n)]
            if not vals:
                raise SystemExit(f"{ctr}: no dispatch of {k} under {d}")
            raw = sum(vals) / len(vals)
            rec = out["per_kernel"].setdefault(k, {})
            rec[ctr.lower() + "_kib_raw"] = round(raw, 1)
            rec[ctr.lower() + "_bytes"] = int(raw * factor * 1024)
            total += raw * factor * 1024
    out["traffic_bytes"] = int(total)
    out["algorithmic_bytes"] = algo_bytes(M, N, K)
    out["source_hash"] = kernel_source_hash()
    return out


def profile_point(workload, M, launches, copy_mib):
    """A short run for counter collection: an optional plain copy of copy_mib MiB (the
    calibration kernel), then `launches` cold launches of one dense point."""
    import torch
    import mxfp4_quantized_gemm_inline_amd as mx
    import workloads as W
    torch.cuda.set_device(0)
    N, K, ms, st = W.DENSE_CONFIGS[workload]
    if copy_mib:
        src = torch.ones(copy_mib << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    wp = mx.mx_prepare_weight(dev_bf16(torch, W.dense_weight(N, K)))
    pt = DensePoint(torch, mx, wp, W.dense_activation(M, K, st), N, K, M, rotate=True)
    torch.cuda.synchronize()
    for i in range(launches):
        pt.launch(i)()
    torch.cuda.synchronize()
    log(f"profiled {workload} M={M}: {launches} launches of "
        f"{mx.mx_a4w4_gemm_plan(M, N, K, mx.mx_a4w4_gemm_workspace_bytes(M, N, K))}")


# ----------------------------------------------------------------------------- CPU baseline

def cpu_baseline(a_by_m, w_bits, ms, n_cols=2048):
    """The oracle as it stands on the host cores, on a bounded sample of one headline step:
    the activations of every M quantized in full, and the weight's first n_cols rows quantized
    and multiplied (decode, float64 matmul) for every M; the weight part is scaled by
    N / n_cols to the whole step (both it and the matmul are linear in the weight rows)."""
    from oracle import mx_oracle as O
    blas = None
    try:
        from threadpoolctl import threadpool_info
        info = threadpool_info()
        blas = max((p.get("num_threads") or 1) for p in info) if info else None
    except Exception:
        blas = None
    cores = len(os.sched_getaffinity(0))
    N = w_bits.shape[0]
    n_cols = min(n_cols, N)
    t0 = time.perf_counter()
    q = {m: O.quantize_mx(a_by_m[m]) for m in ms}
    t_act = time.perf_counter() - t0
    t0 = time.perf_counter()
    qw, sw = O.quantize_mx(w_bits[:n_cols])
    for m in ms:
        O.gemm_from_mx(q[m][0], q[m][1], qw, sw)
    t_w = time.perf_counter() - t0
    step_s = t_act + t_w * N / n_cols
    return {"value": round(step_s * 1e6, 1), "unit": "us/step", "cores": cores, "blas_threads": blas,
            "kind": "oracle",
            "sample": f"one step of N={N} K={w_bits.shape[1]}, M in {list(ms)}: activations quantized in full "
                      f"({t_act:.1f} s), weight rows 0..{n_cols - 1} quantized, decoded and multiplied in float64 "
                      f"for every M ({t_w:.1f} s), scaled by N/{n_cols}; {t_act + t_w:.1f} s of CPU work on "
                      f"{cores} host cores (matmul on {blas} BLAS threads, quantization single-threaded numpy)"}


# ----------------------------------------------------------------------------- main

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-sweep", action="store_true", help="headline step only")
    ap.add_argument("--no-grouped", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--launches", type=int, default=200, help="launches per sweep point")
    ap.add_argument("--profile-point", metavar="WORKLOAD:M",
                    help="counter-collection run: only `--launches` cold launches of this dense point")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="with --profile-point: first run a plain copy of MIB MiB (counter calibration)")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="with --profile-point and --calibrate-copy: turn two rocprofv3 CSV counter "
                         "runs into the calibrated traffic record in profiles/traffic.json")
    args = ap.parse_args()
    if args.profile_point:
        wl, m = args.profile_point.split(":")
        if args.summarize_counters:
            rec = summarize_counters(*args.summarize_counters, wl, int(m), args.calibrate_copy)
            recs = []
            if os.path.exists(TRAFFIC_FILE):
                with open(TRAFFIC_FILE) as f:
                    recs = [r for r in json.load(f)
                            if not (r.get("workload") == wl and r.get("M") == int(m))]
            recs.append(rec)
            with open(TRAFFIC_FILE, "w") as f:
                json.dump(recs, f, indent=1)
            print(json.dumps(rec))
        else:
            profile_point(wl, int(m), args.launches, args.calibrate_copy)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import mxfp4_quantized_gemm_inline_amd as mx
    import workloads as W

    torch.cuda.set_device(0)
    mx.lib()  # fail loudly if the HIP library is missing
    timer = Timer(torch)
    calib = calibrate(torch, mx, timer)
    log(f"calibration: {calib['hbm_read_GBps']:.0f} GB/s streaming read, "
        f"{calib['mfma_fp4_TFLOPs']:.0f} TFLOP/s FP4 MFMA")

    # ---------------- headline: N=8448 K=7168 M sweep, one call per M per step
    N, K, ms, structure = W.DENSE_CONFIGS[HEADLINE]
    w_bits = W.dense_weight(N, K)
    a_all = W.dense_activation(max(ms), K, structure)
    a_by_m = {m: a_all[:m] for m in ms}
    wp = mx.mx_prepare_weight(dev_bf16(torch, w_bits))
    torch.cuda.synchronize()
    log(f"headline {HEADLINE}: prepared weight {wp.numel()} B")
    calib["mfma_fp4_data_TFLOPs"] = calibrate_mfma_data(torch, mx, timer, wp[: N * K // 2], calib["cus"])
    calib.update(calibrate_mfma_clock(torch, mx, wp[: N * K // 2], calib["cus"]))
    calib["mfma_data"] = ("16x16x128 block-scaled FP4 MFMA on the prepared %dx%d weight's own operand bytes, "
                          "one wave per SIMD, 64 accumulators per wave (the register tile of a 128 x 128 wave), "
                          "unit scales" % (N, K))
    log(f"calibration: {calib['mfma_fp4_data_TFLOPs']:.0f} TFLOP/s FP4 MFMA on the weight's own operands")
    log(f"calibration: MFMA loop clock {calib['mfma_clock_GHz_data']:.2f} GHz on the weight's operands "
        f"({calib['mfma_cycles_per_op_data']:.1f} cycles per MFMA), {calib['mfma_clock_GHz_constant']:.2f} GHz "
        f"on constant operands ({calib['mfma_cycles_per_op_constant']:.1f})")

    # rotating sets for the whole step, one graph per set (each holds one step: a call per M)
    per_step = wp.numel() + sum(2 * m * K + 2 * m * N for m in ms)
    R = max(1, min(256, math.ceil(ROTATE_TARGET / per_step)))
    sets = []
    for r in range(R):
        w_r = wp if r == 0 else wp.clone()
        a_r = {m: dev_bf16(torch, a_by_m[m]) for m in ms}
        c_r = {m: torch.empty((m, N), dtype=torch.bfloat16, device="cuda") for m in ms}
        sets.append((w_r, a_r, c_r))

    def step_launches(r):
        w_r, a_r, c_r = sets[r]
        return [(lambda m=m: mx.mx_a4w4_gemm(a_r[m], w_r, N, out=c_r[m])) for m in ms]

    graphs = [timer.graph(step_launches(r)) for r in range(R)]
    for g in graphs:  # first replay of each graph (upload), outside the warmup count
        g.replay()
    for i in range(args.warmup):
        graphs[i % R].replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    t_wall0 = time.perf_counter()
    ev[0].record(stream)
    for i in range(args.steps):
        graphs[i % R].replay()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall0
    per_step_ms = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps))
    step_ms = per_step_ms[len(per_step_ms) // 2]
    mean_ms = ev[0].elapsed_time(ev[-1]) / args.steps
    del graphs
    torch.cuda.empty_cache()
    log(f"headline step: median {step_ms * 1e3:.2f} us/step (mean {mean_ms * 1e3:.2f}, min "
        f"{per_step_ms[0] * 1e3:.2f}, max {per_step_ms[-1] * 1e3:.2f}) over {args.steps} steps, R={R} buffer sets")

    wdev = dev_bf16(torch, w_bits).float()
    head_points = measure_dense(torch, mx, timer, HEADLINE, N, K, ms, wp, a_by_m, wdev, args.launches)
    del wdev
    torch.cuda.empty_cache()
    dom = max(head_points, key=lambda p: p["us"])
    Bd = algo_bytes(dom["M"], N, K)
    Fd = algo_flops(dom["M"], N, K)
    traffic = recorded_traffic(dom["kernel"], HEADLINE, dom["M"])
    if dom["binds"] == "hbm":
        roof = {"bound": "hbm", "achieved": round(Bd / dom["us"] / 1e3, 1), "peak": HBM_PEAK / 1e9,
                "unit": "GB/s", "frac": dom["frac_hbm"], "traffic": traffic}
    else:
        roof = {"bound": "mfma", "achieved": round(Fd / dom["us"] / 1e6, 1), "peak": MFMA_FP4_PEAK / 1e12,
                "unit": "TFLOP/s", "frac": dom["frac_mfma"], "traffic": traffic}
    cal_peak = calib["hbm_read_GBps"] if roof["bound"] == "hbm" else calib["mfma_fp4_data_TFLOPs"]
    roof["peak_calibrated"] = cal_peak
    roof["frac_calibrated"] = round(roof["achieved"] / cal_peak, 4)
    roof["kernel"] = f"{dom['kernel']} (N={N} K={K} M={dom['M']})"
    roof["launch_us"] = dom["us"]
    roof["launch_us_min_max"] = [dom["us_min"], dom["us_max"]]
    roof["duration_note"] = ("one whole GEMM call (every kernel of its plan, back to back on one stream): "
                             f"median over {REPLAYS} replays of a graph of {args.launches} rotated calls, "
                             "HIP events on the replay stream")
    roof["traffic_note"] = ("HBM bytes per call: rocprofv3 FETCH_SIZE and WRITE_SIZE of each kernel of the plan, "
                            "each scaled by its reading on a plain copy of known size (profiles/traffic.json); "
                            "null when the kernel sources changed since the counters were taken")
    roof["algorithmic_bytes"] = Bd
    roof["algorithmic_flops"] = Fd

    # ---------------- full sweep (context)
    sweep = {"dense": [], "grouped": [], "a16w4": []}
    if not args.no_sweep:
        for name, (Nn, Kk, mss, st) in W.DENSE_CONFIGS.items():
            if name in ("smoke_16x256x256", HEADLINE):
                continue
            wb = W.dense_weight(Nn, Kk)
            wpn = mx.mx_prepare_weight(dev_bf16(torch, wb))
            aa = W.dense_activation(max(mss), Kk, st)
            wdn = dev_bf16(torch, wb).float()
            sweep["dense"].extend(measure_dense(torch, mx, timer, name, Nn, Kk, mss, wpn,
                                                {m: aa[:m] for m in mss}, wdn, args.launches))
            del wpn, wdn
            torch.cuda.empty_cache()
        sweep["dense"] = [*head_points, *sweep["dense"]]
        # the A16WFP4 variant (bf16 activations x decoded weight on the bf16 MFMA) at N=7168
        # K=768, the shape of the pages' A16WFP4 call: context, priced against the bf16 MFMA peak
        N16, K16, ms16, st16 = W.DENSE_CONFIGS["n7168_k768"]
        wp16 = mx.mx_prepare_weight(dev_bf16(torch, W.dense_weight(N16, K16)))
        a16 = W.dense_activation(max(ms16), K16, st16)
        for m in ms16:
            cold = DensePoint(torch, mx, wp16, a16[:m], N16, K16, m, rotate=True)

            def launch16(i, pt=cold):
                a_r, w_r, c_r = pt.sets[i % pt.R]
                return lambda: mx.mx_a16w4_gemm(a_r, w_r, N16, out=c_r)
            g = timer.graph([launch16(i) for i in range(args.launches)])
            us16, lo16, hi16 = replay_stats(timer, g, args.launches)
            del g, cold
            Bm, Fm = algo_bytes(m, N16, K16), algo_flops(m, N16, K16)
            sweep["a16w4"].append({"workload": "n7168_k768", "N": N16, "K": K16, "M": m, "us": round(us16, 3),
                                   "us_min": round(lo16, 3), "us_max": round(hi16, 3),
                                   "tflops": round(Fm / us16 / 1e6, 2), "gbps": round(Bm / us16 / 1e3, 1),
                                   "frac_hbm": round(Bm / HBM_PEAK * 1e6 / us16, 4),
                                   "frac_mfma_bf16": round(Fm / MFMA_BF16_PEAK * 1e6 / us16, 4),
                                   "kernel": mx.mx_a16w4_gemm_plan(m, N16, K16)})
            log(f"  a16w4 n7168_k768 M={m}: {us16:.2f} us cold")
        del wp16
        if not args.no_grouped:
            sweep["grouped"] = grouped_sweep(torch, mx, W, timer)

    # every point's binding fraction against the measured ceilings as well
    for p in [*head_points, *sweep["dense"], *sweep["grouped"]]:
        if "us" in p and "N" in p and "K" in p and "M" in p:
            Bp, Fp = algo_bytes(p["M"], p["N"], p["K"]), algo_flops(p["M"], p["N"], p["K"])
        elif "bytes" in p and "flops" in p:
            Bp, Fp = p["bytes"], p["flops"]
        else:
            continue
        p["frac_binding_calibrated"] = round(max(Bp / calib["hbm_read_GBps"] / 1e3,
                                                 Fp / calib["mfma_fp4_data_TFLOPs"] / 1e6) / p["us"], 4)

    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(a_by_m, w_bits, ms)
        log(f"cpu oracle: {cpu['value']:.0f} us/step")

    page_total = sum(PAGE_US[(HEADLINE, m)] for m in ms)
    value = step_ms * 1e3
    out = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "us/step",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 6),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": round(value / page_total, 4),
        "dtype": "mxfp4",
        "data": "synthetic",
        "config": {"workload": f"dense A4W4 MXFP4 GEMM N={N} K={K}, one call per M in {list(ms)} per step",
                   "N": N, "K": K, "M": list(ms), "buffer_sets": R,
                   "a": "bf16 ~N(0,1); in 0.5% of rows (row 0 among them) each 32-block zeroed with "
                        "probability 1/4, the first as -0",
                   "w": "bf16 ~N(0,0.02) prepared to MXFP4",
                   "timing": "one HIP graph replay per step, HIP events between steps; median step; "
                             "rotating buffer sets > Infinity Cache"},
        "step_us": {"median": round(value, 3), "mean": round(mean_ms * 1e3, 3),
                    "min": round(per_step_ms[0] * 1e3, 3), "max": round(per_step_ms[-1] * 1e3, 3),
                    "p10": round(per_step_ms[len(per_step_ms) // 10] * 1e3, 3),
                    "p90": round(per_step_ms[(9 * len(per_step_ms)) // 10] * 1e3, 3)},
        "baseline_note": f"vs_baseline = value / {page_total:.3f} us, the sum of the pages' direct-kernel "
                         f"medians for this sweep on MI355X (lower is better)",
        "roofline": roof,
        "calibration": calib,
        "cpu_baseline": cpu,
        "points": head_points,
        "sweep": sweep,
        "wall_s_timed": round(t_wall, 4),
    }
    print(json.dumps(out), flush=True)


def measure_dense(torch, mx, timer, name, N, K, ms, wp, a_by_m, w_f32, launches):
    """Cold (rotated) and warm (one set) time per M, and the relative L2 of the output against
    the unquantized product: ||C - A W^T|| / ||A W^T|| with A and W the bf16 inputs, the
    reference in fp32 on the GPU (context only: the parity tests compare with the oracle)."""
    recs = []
    for m in ms:
        cold = DensePoint(torch, mx, wp, a_by_m[m], N, K, m, rotate=True)
        us_c = time_point(timer, cold, launches)
        a0, w0, c0 = cold.sets[0]
        ref = a0.float() @ w_f32.t()
        rel = float(torch.linalg.vector_norm(c0.float() - ref) / torch.linalg.vector_norm(ref))
        del cold, ref
        warm = DensePoint(torch, mx, wp, a_by_m[m], N, K, m, rotate=False)
        us_w = time_point(timer, warm, launches)[0]
        del warm
        rec = point_record(name, N, K, m, us_c, us_w, kernel_name(mx, m, N, K))
        rec["rel_l2_vs_bf16"] = round(rel, 5)
        recs.append(rec)
        log(f"  {name} M={m}: {us_c[0]:.2f} us cold ({us_c[1]:.2f}..{us_c[2]:.2f}), {us_w:.2f} us warm, "
            f"rel-L2 {rel:.4f}")
    return recs


def grouped_sweep(torch, mx, W, timer):
    """The MoE layer at T = 1, 16, 256, 4096 (E=896, top-16): grouped GEMM1 (K=3584, N=1536)
    with bf16 output and with the fused SwiGLU + MXFP4 epilogue, the second GEMM on MXFP4 rows
    (K=768, N=3584) and the top-16 combine."""
    N, K, E = W.MOE_N, W.MOE_K, W.MOE_E
    per = mx.mx_prepared_weight_bytes(N, K)
    stack = torch.empty(E * per, dtype=torch.uint8, device="cuda")
    t0 = time.perf_counter()
    for e, w in W.moe_expert_weights(range(E), threads=min(16, os.cpu_count() or 8)):
        mx.mx_prepare_weight(dev_bf16(torch, w), out=stack[e * per:(e + 1) * per])
    per2 = mx.mx_prepared_weight_bytes(W.MOE_N2, W.MOE_K2)
    stack2 = torch.empty(E * per2, dtype=torch.uint8, device="cuda")
    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(min(16, os.cpu_count() or 8)) as ex:
        for e, w2 in zip(range(E), ex.map(W.moe_expert_weight2, range(E))):
            mx.mx_prepare_weight(dev_bf16(torch, w2), out=stack2[e * per2:(e + 1) * per2])
    torch.cuda.synchronize()
    log(f"grouped: prepared {E} experts (both GEMMs) in {time.perf_counter() - t0:.1f} s")
    recs = []
    for T in W.MOE_TOKENS:
        a = dev_bf16(torch, W.moe_activation(T))
        _, offs, row_token = W.moe_routing(T)
        R = int(offs[-1])
        active = int((offs[1:] > offs[:-1]).sum())
        hint = max(1, -(-R // min(E, R)))
        rt = torch.from_numpy(row_token).cuda()
        of = torch.from_numpy(offs).cuda()
        c = torch.empty((R, N), dtype=torch.bfloat16, device="cuda")
        n = 20 if T >= 256 else 100
        g = timer.graph([lambda: mx.mx_a4w4_gemm_grouped(a, rt, of, E, R, stack, N, rows_hint=hint, out=c)] * n)
        us = timer.replay_ms(g, reps=2) * 1e3 / n
        del g
        B = active * per + 2 * T * K + 2 * R * N
        F = 2 * R * N * K
        recs.append({"workload": "grouped_moe_gemm1_e896_top16_k3584_n1536", "T": T, "rows": R,
                     "active_experts": active, "us": round(us, 3), "bytes": B, "flops": F,
                     "tflops": round(F / us / 1e6, 2), "gbps": round(B / us / 1e3, 1),
                     "frac_hbm": round(B / HBM_PEAK * 1e6 / us, 4),
                     "frac_mfma": round(F / MFMA_FP4_PEAK * 1e6 / us, 4),
                     "kernel": mx.mx_a4w4_gemm_grouped_plan(E, R, T, N, K, hint)})
        log(f"  grouped T={T}: {us:.2f} us ({active} experts, {R} rows)")
        # the same GEMM1 with the fused SwiGLU + MXFP4 epilogue: h [R, N/2] as E2M1 + E8M0
        Nh = N // 2
        hq = torch.empty((R, Nh // 2), dtype=torch.uint8, device="cuda")
        hs = torch.empty((R, Nh // 32), dtype=torch.uint8, device="cuda")
        g = timer.graph([lambda: mx.mx_a4w4_gemm_grouped_act_quant(a, rt, of, E, R, stack, N, act=mx.MX_ACT_SWIGLU,
                                                                   rows_hint=hint, h_fp4=hq, h_scale=hs)] * n)
        us_f = timer.replay_ms(g, reps=2) * 1e3 / n
        del g, hq, hs
        Bf = active * per + 2 * T * K + R * (Nh // 2 + Nh // 32)
        recs.append({"workload": "grouped_moe_gemm1_swiglu_mxfp4_e896_top16_k3584_n1536", "T": T, "rows": R,
                     "active_experts": active, "us": round(us_f, 3), "bytes": Bf, "flops": F,
                     "tflops": round(F / us_f / 1e6, 2), "gbps": round(Bf / us_f / 1e3, 1),
                     "frac_hbm": round(Bf / HBM_PEAK * 1e6 / us_f, 4),
                     "frac_mfma": round(F / MFMA_FP4_PEAK * 1e6 / us_f, 4),
                     "kernel": mx.mx_a4w4_gemm_grouped_act_quant_plan(E, R, N, K, mx.MX_ACT_SWIGLU, hint)})
        log(f"  grouped T={T} + fused SwiGLU/MXFP4 epilogue: {us_f:.2f} us")
        # the layer's second GEMM on MXFP4 rows (inter_dim 768 -> model_dim 3584), then the combine
        N2, K2 = W.MOE_N2, W.MOE_K2
        aq_h, as_h = W.mx_bytes(R, K2, seed=500 + T)
        aq, as_ = torch.from_numpy(aq_h).cuda(), torch.from_numpy(as_h).cuda()
        y = torch.empty((R, N2), dtype=torch.bfloat16, device="cuda")
        g = timer.graph([lambda: mx.mx_a4w4_gemm_grouped_mx(aq, as_, of, E, R, stack2, N2, rows_hint=hint, out=y)] * n)
        us2 = timer.replay_ms(g, reps=2) * 1e3 / n
        del g
        B2 = active * per2 + R * (K2 // 2 + K2 // 32) + 2 * R * N2
        F2 = 2 * R * N2 * K2
        recs.append({"workload": "moe_gemm2_mxfp4_e896_top16_k768_n3584", "T": T, "rows": R, "active_experts": active,
                     "us": round(us2, 3), "bytes": B2, "flops": F2, "tflops": round(F2 / us2 / 1e6, 2),
                     "gbps": round(B2 / us2 / 1e3, 1), "frac_hbm": round(B2 / HBM_PEAK * 1e6 / us2, 4),
                     "frac_mfma": round(F2 / MFMA_FP4_PEAK * 1e6 / us2, 4),
                     "kernel": mx.mx_a4w4_gemm_grouped_mx_plan(N2, K2, hint)})
        tr = torch.from_numpy(W.moe_token_rows(W.moe_routing(T)[0])).cuda()
        wt = torch.from_numpy(W.moe_combine_weights(T)).cuda()
        o = torch.empty((T, N2), dtype=torch.bfloat16, device="cuda")
        g = timer.graph([lambda: mx.mx_moe_combine(y, tr, wt, out=o)] * n)
        us_c = timer.replay_ms(g, reps=2) * 1e3 / n
        del g, y, o, aq, as_
        Bc = 2 * R * N2 + 2 * T * N2 + 8 * R
        recs.append({"workload": "moe_combine_top16_n3584", "T": T, "rows": R, "us": round(us_c, 3), "bytes": Bc,
                     "flops": 2 * R * N2, "gbps": round(Bc / us_c / 1e3, 1),
                     "frac_hbm": round(Bc / HBM_PEAK * 1e6 / us_c, 4), "kernel": "k_moe_combine"})
        log(f"  T={T} second GEMM on MXFP4 rows: {us2:.2f} us; top-16 combine: {us_c:.2f} us")
    del stack, stack2
    torch.cuda.empty_cache()
    return recs


if __name__ == "__main__":
    main()
