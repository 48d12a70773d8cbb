#!/usr/bin/env python3
"""Benchmark of the fused fp32 convolutions on one MI355X.

One step = one call of each fused kernel on its full-size workload, inputs
already resident in HBM:
  * fconv2d_pool_sigmoid_sum on x[128,8,384,384], Conv2d 8->64 k3, AvgPool 4,
    with the direct convolution the method defines (FCONV_ALGO_DIRECT_MFMA)
  * dwsep_conv1d on x[32,256,4096], depthwise k9 pad 4, pointwise 256->512
Untimed whole steps run for --settle-s seconds first (the clocks ramp up from
idle over tens of milliseconds), then --warmup untimed steps, then --steps
timed ones.  Prints one JSON line (driver contract) with whole-step GFLOP/s, per-kernel
ms/call and GFLOP/s, the roofline fraction of the dominant kernel, and the CPU
oracle timed on a bounded sample of the same workloads.

`configs` reports every workload (the two small ones, the two full-size ones
and the K5/s3 one) through the entry points' default algorithm (AUTO) and,
for the Conv2d workloads, the direct one: ms per call as the median, p10 and
p90 of repeated runs of back-to-back calls between one event pair, GFLOP/s,
a roofline, and the largest error against the oracle as a fraction of the
1e-4 tolerance, with the oracle's wall time.

FLOPs are algorithmic, 2 per multiply-add: the conv outputs that feed the pool,
s*s*Cin*K*K MACs per (co, pooled output); the separable conv1d, C*K + O*C MACs
per time step (not the dense fused form).
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import fconv_inputs as fi  # noqa: E402

METRIC = "fp32 GFLOP/s + ms/call per fused conv; fraction of MI355X fp32 roofline"
PEAK_FP32_TFLOPS = 157.3  # MI355X dense fp32 (matrix cores), published
PEAK_HBM_GBPS = 8000.0

CONV = "conv2d_full"
TAIL = "conv2d_tail"
DW = "dwsep_full"

TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")
# Sources that define the timed kernels; measured HBM traffic is reported
# only while their hash matches the one recorded with the counters.
# Keys are kernel-name parts as rocprofv3 prints them; the template arguments
# of conv2d_pool_elem_kernel are <tiling <K, s, column blocks, pooled rows>,
# pool (0 mean, 1 max, 2 mean with the rows folded into the MFMAs), output mode,
# channel quads with weights resident in registers (0: streamed), whether
# each workgroup walks several tiles>.
KERNEL_SOURCES = {
    "conv2d_pool_elem_kernel<fconv::ElemCfg<3, 4, 4, 3, false>, 2, 2, 2, false>": [
        "fp32_convolution_amd/csrc/conv2d_pool_ex.hip", "fp32_convolution_amd/csrc/fconv_device.hpp"],
    "dwsep_tall_kernel<fconv::DwsepCfg<4, 4, 8, 1, 64, 9, 4>, 1, 0>": ["fp32_convolution_amd/csrc/dwsep_conv1d.hip",
                                                                    "fp32_convolution_amd/csrc/fconv_device.hpp"],
    "conv2d_pool_boxsum4_kernel<2, true, 2, false>": ["fp32_convolution_amd/csrc/conv2d_pool.hip",
                                                      "fp32_convolution_amd/csrc/fconv_device.hpp"],
    "conv2d_pool_boxsum_kernel<fconv::DirectCfg<5, 3, 1, 3, 8, 1, 4, 12>, 2, false>": [
        "fp32_convolution_amd/csrc/conv2d_pool.hip", "fp32_convolution_amd/csrc/fconv_device.hpp"],
    "dwsep_dense_kernel": ["fp32_convolution_amd/csrc/dwsep_conv1d.hip",
                           "fp32_convolution_amd/csrc/fconv_device.hpp"],
    "conv2d_pool_elem_kernel<fconv::ElemCfg<3, 4, 4, 4, false>, 1, 2, 2, false>": [
        "fp32_convolution_amd/csrc/conv2d_pool_ex.hip", "fp32_convolution_amd/csrc/fconv_device.hpp"],
    "conv2d_pool_mfma_kernel<fconv::DirectCfg<5, 3, 1, 3, 8, 1, 4, 12>, 2, false>": [
        "fp32_convolution_amd/csrc/conv2d_pool.hip", "fp32_convolution_amd/csrc/fconv_device.hpp"],
}


ELEM_AVG = "conv2d_pool_elem_kernel<fconv::ElemCfg<3, 4, 4, 3, false>, 2, 2, 2, false>"
# the separable dwsep kernel of the step: the 512 x 64 tile, K = 9, stride 1
DW_TALL = "dwsep_tall_kernel<fconv::DwsepCfg<4, 4, 8, 1, 64, 9, 4>, 1, 0>"
ELEM_MAX = "conv2d_pool_elem_kernel<fconv::ElemCfg<3, 4, 4, 4, false>, 1, 2, 2, false>"
TRACE_FILE = os.path.join(ROOT, "profiles", "kernel_trace.json")


def sources_sha256(kernel):
    import hashlib

    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def trace_kernel_ms(kernel):
    """Average kernel duration (ms) from the recorded rocprofv3 kernel trace,
    or None if missing or the kernel's sources changed since."""
    try:
        with open(TRACE_FILE) as f:
            rec = json.load(f)["kernels"][kernel]
    except (OSError, KeyError, ValueError):
        return None
    if rec.get("sources_sha256") != sources_sha256(kernel):
        return None
    return rec["average_ms"]


def ingest_trace(stats_csv, command):
    """Writes TRACE_FILE from a rocprofv3 --kernel-trace --stats run: the
    average duration of each kernel in KERNEL_SOURCES (first matching name)."""
    import csv

    rows = list(csv.DictReader(open(stats_csv)))
    out = {"command": command, "kernels": {}}
    for kernel in KERNEL_SOURCES:
        hit = [r for r in rows if kernel in r["Name"]]
        if not hit:
            continue
        r = max(hit, key=lambda r: int(r["Calls"]))
        out["kernels"][kernel] = {"kernel_name": r["Name"], "calls": int(r["Calls"]),
                                  "average_ms": round(float(r["AverageNs"]) / 1e6, 5),
                                  "sources_sha256": sources_sha256(kernel)}
    with open(TRACE_FILE, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out, indent=1))


def measured_traffic(kernel):
    """HBM bytes per launch from the recorded counters, or None if the record
    is missing or the kernel's sources changed since it was taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)["kernels"][kernel]
    except (OSError, KeyError, ValueError):
        return None
    if rec.get("sources_sha256") != sources_sha256(kernel):
        return None
    return rec["hbm_bytes_per_launch"]


def ingest_counters(fetch_csv, write_csv, copy_mb, command):
    """Writes TRAFFIC_FILE from two rocprofv3 --pmc runs of this script with
    --copy-calibration-mb: FETCH_SIZE and WRITE_SIZE (KiB per dispatch) of each
    timed kernel, scaled by what the same counters read for the calibration
    copy of copy_mb MiB (which reads and writes exactly that many bytes)."""
    import csv

    def per_kernel(path, counter):
        vals = {}
        with open(path) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] != counter:
                    continue
                vals.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        return vals

    fetch = per_kernel(fetch_csv, "FETCH_SIZE")
    write = per_kernel(write_csv, "WRITE_SIZE")
    copy_kib = copy_mb * 1024.0
    cal_f = [v for k, vs in fetch.items() if "copyBuffer" in k for v in vs if v > 0.25 * copy_kib]
    cal_w = [v for k, vs in write.items() if "copyBuffer" in k for v in vs if v > 0.25 * copy_kib]
    if not cal_f or not cal_w:
        raise SystemExit("calibration copy not found in the counter files")
    f_scale, w_scale = copy_kib / max(cal_f), copy_kib / max(cal_w)
    out = {"fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4),
           "calibration": f"device copy of {copy_mb} MiB: FETCH_SIZE {max(cal_f):.1f} KiB, "
                          f"WRITE_SIZE {max(cal_w):.1f} KiB",
           "command": command, "kernels": {}}
    for kernel in KERNEL_SOURCES:
        fk = [v for k, vs in fetch.items() if kernel in k for v in vs]
        wk = [v for k, vs in write.items() if kernel in k for v in vs]
        if not fk or not wk:
            continue
        fb = sum(fk) / len(fk) * 1024 * f_scale
        wb = sum(wk) / len(wk) * 1024 * w_scale
        name = next(k for k in fetch if kernel in k)
        out["kernels"][kernel] = {"kernel_name": name, "dispatches": len(fk),
                                  "fetch_kib_raw": round(sum(fk) / len(fk), 1),
                                  "write_kib_raw": round(sum(wk) / len(wk), 1),
                                  "hbm_read_bytes_per_launch": int(fb), "hbm_write_bytes_per_launch": int(wb),
                                  "hbm_bytes_per_launch": int(fb + wb),
                                  "sources_sha256": sources_sha256(kernel)}
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out, indent=1))


PROBE_LIB = os.path.join(ROOT, "fp32_convolution_amd", "libfconv_probe.so")


def measured_ceilings(torch, dev, stream):
    """What the GPU sustains for each bound, measured here (libfconv_probe.so):
    the fp32 matrix-core rate and the non-packed fp32 vector FMA rate (eight
    independent chains of one instruction per wave, best of 1, 2 and 4 waves
    per SIMD), a 1 GiB streaming read, a 1 GiB streaming write and a 1 GiB
    device-to-device copy (read + write bytes).  Each timing is the median of
    5 launches after 2 untimed ones."""
    import ctypes

    def med_ms(launch):
        ms = []
        for i in range(7):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            launch()
            e1.record(stream)
            torch.cuda.synchronize()
            if i >= 2:
                ms.append(e0.elapsed_time(e1))
        return float(np.median(ms))

    res = {}
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    n = (1 << 30) // 4
    if os.path.exists(PROBE_LIB):
        lib = ctypes.CDLL(PROBE_LIB)
        out = torch.empty(cus * 8 * 256, device=dev)
        st = ctypes.c_void_p(stream.cuda_stream)
        for name, fn, flop_per_inst, iters in (
                ("mfma_f32_16x16x4", lib.fconv_probe_mfma_f32, 2 * 16 * 16 * 4, 4000),
                ("valu_fma_f32", lib.fconv_probe_fma_f32, 2 * 64, 40000)):
            fn.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
            best = 0.0
            for wps in (1, 2, 4):
                blocks = cus * wps

                def launch():
                    if fn(blocks, iters, ctypes.c_void_p(out.data_ptr()), st) != 0:
                        raise RuntimeError(f"probe {name} failed to launch")

                flops = flop_per_inst * 8 * iters * blocks * 4
                best = max(best, flops / (med_ms(launch) * 1e-3) / 1e12)
            res[name] = {"tflops": round(best, 1)}
        res["mfma_f32_16x16x4"].update({"peak": PEAK_FP32_TFLOPS,
                                        "frac_of_peak": round(res["mfma_f32_16x16x4"]["tflops"] / PEAK_FP32_TFLOPS, 4)})
        # The datasheet's 78.6 TFLOP/s for non-packed fp32 assumes one wave64
        # v_fma_f32 per SIMD every 4 cycles at 2.4 GHz; the probe issues them
        # faster than that, so the figure is a nominal rate, not a ceiling.
        # Recorded: the measured rate and the cycles per wave instruction it
        # implies at 2.4 GHz.
        v = res["valu_fma_f32"]["tflops"]
        res["valu_fma_f32"].update({
            "nominal_non_packed_tflops": 78.6,
            "implied_cycles_per_wave64_fma_at_2400MHz": round(cus * 4 * 2.4e9 * 128 / (v * 1e12), 2)})
        # vector work beside matrix work on one SIMD: overlapped or in turn
        fn = lib.fconv_probe_mfma_valu_f32
        fn.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
        ov = torch.empty(cus * 512, device=dev)
        t_mode = {}
        for mode in (1, 2, 3):
            def launch_ov(mode=mode):
                if fn(cus, mode, 4000, 15000, ctypes.c_void_p(ov.data_ptr()), st) != 0:
                    raise RuntimeError("probe mfma_valu failed to launch")
            t_mode[mode] = med_ms(launch_ov)
        res["mfma_beside_valu"] = {
            "mfma_waves_ms": round(t_mode[1], 4), "valu_waves_ms": round(t_mode[2], 4), "both_ms": round(t_mode[3], 4),
            "overlap": round((t_mode[1] + t_mode[2] - t_mode[3]) / min(t_mode[1], t_mode[2]), 3),
            "what": "one wave of v_mfma_f32_16x16x4_f32 chains and one of v_fma_f32 chains per SIMD; overlap 1 = "
                    "both-mode time is the longer of the two, 0 = their sum (the SIMD runs them in turn)"}
        del ov
        src = torch.ones(n, device=dev)
        red = torch.empty(cus * 8 * 256, device=dev)
        lib.fconv_probe_read_f32.argtypes = [ctypes.c_int, ctypes.c_long, ctypes.c_void_p, ctypes.c_void_p,
                                             ctypes.c_void_p]
        lib.fconv_probe_write_f32.argtypes = [ctypes.c_int, ctypes.c_long, ctypes.c_void_p, ctypes.c_void_p]
        best_r = best_w = 0.0
        for wps in (2, 4, 8):
            blocks = cus * wps
            tr = med_ms(lambda: lib.fconv_probe_read_f32(blocks, n // 4, ctypes.c_void_p(src.data_ptr()),
                                                         ctypes.c_void_p(red.data_ptr()), st))
            tw = med_ms(lambda: lib.fconv_probe_write_f32(blocks, n // 4, ctypes.c_void_p(src.data_ptr()), st))
            best_r = max(best_r, n * 4 / (tr * 1e-3) / 1e9)
            best_w = max(best_w, n * 4 / (tw * 1e-3) / 1e9)
        res["hbm_read"] = {"gbps": round(best_r, 1), "peak": PEAK_HBM_GBPS, "frac_of_peak": round(best_r / PEAK_HBM_GBPS, 4),
                           "what": "1 GiB streaming read, 16-byte loads, best of 2, 4, 8 workgroups per CU"}
        res["hbm_write"] = {"gbps": round(best_w, 1), "peak": PEAK_HBM_GBPS,
                            "frac_of_peak": round(best_w / PEAK_HBM_GBPS, 4),
                            "what": "1 GiB streaming write, 16-byte stores, best of 2, 4, 8 workgroups per CU"}
        del out, src, red
    src = torch.ones(n, device=dev)
    dst = torch.empty_like(src)
    gbps = 2 * n * 4 / (med_ms(lambda: dst.copy_(src)) * 1e-3) / 1e9
    res["hbm_copy"] = {"gbps": round(gbps, 1), "peak": PEAK_HBM_GBPS, "frac_of_peak": round(gbps / PEAK_HBM_GBPS, 4),
                       "what": "1 GiB device-to-device copy (torch), read + write bytes"}
    del src, dst
    return res


def conv2d_flops(cfg):
    Hc, Wc = cfg["H"] - cfg["K"] + 1, cfg["W"] - cfg["K"] + 1
    s = cfg["pool"]
    PH, PW = Hc // s, Wc // s
    return 2 * cfg["B"] * cfg["Cout"] * PH * PW * s * s * cfg["Cin"] * cfg["K"] ** 2


def conv2d_boxsum_flops(cfg):
    """Work of the box-sum form: Cin*K*K MACs per (co, pooled output)."""
    Hc, Wc = cfg["H"] - cfg["K"] + 1, cfg["W"] - cfg["K"] + 1
    s = cfg["pool"]
    PH, PW = Hc // s, Wc // s
    return 2 * cfg["B"] * cfg["Cout"] * PH * PW * cfg["Cin"] * cfg["K"] ** 2


def conv2d_bytes(cfg):
    return 4 * (cfg["B"] * cfg["Cin"] * cfg["H"] * cfg["W"] + cfg["Cout"] * cfg["Cin"] * cfg["K"] ** 2
                + cfg["Cout"] + cfg["B"])


def dwsep_flops(cfg):
    Tout = cfg["T"] + 2 * cfg["pad"] - cfg["K"] + 1
    return 2 * cfg["B"] * Tout * cfg["C"] * (cfg["K"] + cfg["O"])


def dwsep_dense_flops(cfg):
    """Work of the dense-fused form: C*K*O MACs per output step."""
    Tout = cfg["T"] + 2 * cfg["pad"] - cfg["K"] + 1
    return 2 * cfg["B"] * Tout * cfg["C"] * cfg["K"] * cfg["O"]


def dwsep_bytes(cfg):
    Tout = cfg["T"] + 2 * cfg["pad"] - cfg["K"] + 1
    return 4 * (cfg["B"] * cfg["C"] * cfg["T"] + cfg["C"] * cfg["K"] + cfg["O"] * cfg["C"] + cfg["O"]
                + cfg["B"] * cfg["O"] * Tout)


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            return next(line.split(":", 1)[1].strip() for line in f if line.startswith("model name"))
    except (OSError, StopIteration):
        return "unknown"


def err_over_tol(got, want):
    """Largest |gpu - oracle| / (1e-4 + 1e-4 |oracle|): at most 1 within the specified tolerance."""
    got = np.asarray(got, dtype=np.float64)
    return float((np.abs(got - want) / (1e-4 + 1e-4 * np.abs(want))).max())


def abs_rel_err(got, want):
    """Largest |gpu - oracle|, and largest |gpu - oracle| / |oracle| over the outputs with
    |oracle| >= 1e-4 (below that the tolerance's absolute term governs)."""
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    d = np.abs(got - want)
    big = np.abs(want) >= 1e-4
    return float(d.max()), (float((d[big] / np.abs(want[big])).max()) if big.any() else 0.0)


ALGO_NAMES = {0: "FCONV_ALGO_AUTO", 1: "FCONV_ALGO_DIRECT_MFMA", 2: "FCONV_ALGO_DIRECT_SIMPLE", 3: "FCONV_ALGO_BOXSUM"}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--settle-s", type=float, default=0.3,
                    help="untimed whole steps run first for this long, so that the clocks have left their idle state")
    ap.add_argument("--reps", type=int, default=20, help="timed repetitions per call in `configs` and `variants`")
    ap.add_argument("--per-rep", type=int, default=10, help="back-to-back calls between one event pair")
    ap.add_argument("--call-warm-s", type=float, default=0.05,
                    help="untimed calls of the same call for at least this long before its timed runs in `configs` "
                         "and `variants`, so that the clocks leave the state the previous (lighter or idle) work left")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle timing and parity legs")
    ap.add_argument("--copy-calibration-mb", type=int, default=0,
                    help="run one device copy of this many MiB first (reference for HBM byte counters)")
    ap.add_argument("--ingest-counters", nargs=3, metavar=("FETCH_CSV", "WRITE_CSV", "COPY_MB"),
                    help="write profiles/hbm_traffic.json from rocprofv3 counter files and exit")
    ap.add_argument("--ingest-trace", metavar="KERNEL_STATS_CSV",
                    help="write profiles/kernel_trace.json from a rocprofv3 --kernel-trace --stats file and exit")
    ap.add_argument("--ingest-command", default="", help="the profiling command, recorded with the counters")
    args = ap.parse_args()

    if args.ingest_counters:
        fetch_csv, write_csv, copy_mb = args.ingest_counters
        ingest_counters(fetch_csv, write_csv, int(copy_mb), args.ingest_command)
        return
    if args.ingest_trace:
        ingest_trace(args.ingest_trace, args.ingest_command)
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: every kernel here runs on a single device and the "
              "multi-GPU sharding is a design note, not an implementation. Run with --gpus 1.",
              file=sys.stderr, flush=True)
        sys.exit(2)

    import torch

    import fp32_convolution_amd as fc

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)

    host = {name: fi.make(name, seed=args.seed) for name in fi.WORKLOADS}
    gpu = {name: [torch.from_numpy(a).to(dev) for a in arrs] for name, arrs in host.items()}
    cc, dc, tc = fi.WORKLOADS[CONV], fi.WORKLOADS[DW], fi.WORKLOADS[TAIL]
    x, w, b = gpu[CONV]
    xd, wdw, wpw, bpw = gpu[DW]
    out = torch.empty(cc["B"], device=dev)
    Tout = fc.dwsep_out_len(dc["T"], dc["K"], dc["pad"])
    y = torch.empty((dc["B"], dc["O"], Tout), device=dev)

    if args.copy_calibration_mb > 0:
        n = args.copy_calibration_mb * (1 << 20) // 4
        src = torch.ones(n, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    def conv_call():
        fc.conv2d_pool_sigmoid_sum(x, w, b, cc["pool"], out=out, algo=fc.ALGO_DIRECT_MFMA)

    def dw_call():
        fc.dwsep_conv1d(xd, wdw, wpw, bpw, dc["pad"], out=y)

    # From idle the clocks take tens of milliseconds to ramp up: per-call
    # times fall by about 20 % over the first 15 steps.  Untimed steps run
    # for settle_s first, then the warm-up steps, then the timed ones.
    t_settle = time.perf_counter()
    settle_steps = 0
    while True:
        for _ in range(10):
            conv_call()
            dw_call()
        settle_steps += 10
        torch.cuda.synchronize()
        if time.perf_counter() - t_settle >= args.settle_s:
            break
    t_settle = time.perf_counter() - t_settle
    for _ in range(args.warmup):
        conv_call()
        dw_call()
    torch.cuda.synchronize()

    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    start.record(stream)
    for e in ev:
        e[0].record(stream)
        conv_call()
        e[1].record(stream)
        dw_call()
        e[2].record(stream)
    end.record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall

    def time_calls(fn):
        """ms per call: `reps` runs of `per_rep` back-to-back calls, each run
        between one event pair (so host time between calls is hidden as it
        is in a stream of calls), after untimed runs of the same call for at
        least `call_warm_s` seconds (after the host-side oracle or a few
        microsecond-long calls, 10 calls left the box-sum call on
        x[128,8,384,384] 4-8 % slower than in a steady stream)."""
        for _ in range(args.per_rep):
            fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < args.call_warm_s:
            for _ in range(args.per_rep):
                fn()
            torch.cuda.synchronize()
        evs = []
        for _ in range(args.reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(args.per_rep):
                fn()
            e1.record(stream)
            evs.append((e0, e1))
        torch.cuda.synchronize()
        return np.array([e0.elapsed_time(e1) / args.per_rep for e0, e1 in evs])

    def stats(ms):
        return {"ms_mean": round(float(ms.mean()), 4), "ms_median": round(float(np.median(ms)), 4),
                "ms_p10": round(float(np.percentile(ms, 10)), 4), "ms_p90": round(float(np.percentile(ms, 90)), 4)}

    def roofline(bound, work, ms):
        if bound == "mfma":
            a = work / (ms * 1e-3) / 1e12
            return {"bound": "mfma", "achieved": round(a, 2), "peak": PEAK_FP32_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(a / PEAK_FP32_TFLOPS, 4)}
        a = work / (ms * 1e-3) / 1e9
        return {"bound": "hbm", "achieved": round(a, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                "frac": round(a / PEAK_HBM_GBPS, 4)}

    # ---- every workload through the entry points' default algorithm (and the
    #      direct one for the Conv2d workloads)
    conv_outputs, dw_outputs = {}, {}
    configs = {}
    for name, cfg in fi.WORKLOADS.items():
        ent = {"shape": {k: v for k, v in cfg.items() if k != "kind"}}
        if cfg["kind"] == "conv2d":
            xx, ww, bb = gpu[name]
            f_method, nbytes = conv2d_flops(cfg), conv2d_bytes(cfg)
            ent["algorithmic_gflop"] = round(f_method / 1e9, 6)
            ent["algorithmic_bytes"] = nbytes
            auto = fc.conv2d_select_algo(cfg["Cin"], cfg["Cout"], cfg["K"], cfg["pool"])
            algos = [(0, auto)] + ([(fc.ALGO_DIRECT_MFMA, fc.ALGO_DIRECT_MFMA)]
                                   if auto != fc.ALGO_DIRECT_MFMA and cfg["B"] > 2 else [])
            for call_algo, runs in algos:
                o = torch.empty(cfg["B"], device=dev)
                ms = time_calls(lambda: fc.conv2d_pool_sigmoid_sum(xx, ww, bb, cfg["pool"], out=o, algo=call_algo))
                torch.cuda.synchronize()
                own = conv2d_boxsum_flops(cfg) if runs == fc.ALGO_BOXSUM else f_method
                m = float(np.median(ms))
                e = stats(ms)
                e["algorithm"] = ALGO_NAMES[runs] + (" (the default, AUTO)" if call_algo == 0 else "")
                e["own_gflop"] = round(own / 1e9, 6)
                e["gflops_own"] = round(own / (m * 1e-3) / 1e9, 1)
                e["hbm_gbps_algorithmic"] = round(nbytes / (m * 1e-3) / 1e9, 1)
                # the box-sum form's own work sits near or below the ridge point
                # (17.6 FLOP/B for K3/s4): its roofline is the larger of the two times
                bound = "mfma" if own / nbytes > PEAK_FP32_TFLOPS * 1e12 / (PEAK_HBM_GBPS * 1e9) else "hbm"
                e["roofline"] = roofline(bound, own if bound == "mfma" else nbytes, m)
                if cfg["B"] <= 4:
                    e["roofline"]["note"] = "launch-bound: the whole call is a few microseconds of launch overhead"
                ent["default" if call_algo == 0 else "direct_mfma"] = e
                conv_outputs[(name, call_algo)] = o.cpu().numpy().astype(np.float64)
        else:
            xx, wd_, wp_, bp_ = gpu[name]
            To = fc.dwsep_out_len(cfg["T"], cfg["K"], cfg["pad"])
            yy = torch.empty((cfg["B"], cfg["O"], To), device=dev)
            f_method, nbytes = dwsep_flops(cfg), dwsep_bytes(cfg)
            ent["algorithmic_gflop"] = round(f_method / 1e9, 6)
            ent["algorithmic_bytes"] = nbytes
            ms = time_calls(lambda: fc.dwsep_conv1d(xx, wd_, wp_, bp_, cfg["pad"], out=yy))
            m = float(np.median(ms))
            e = stats(ms)
            e["algorithm"] = "FCONV_DWSEP_SEPARABLE (the default)"
            e["gflops_own"] = round(f_method / (m * 1e-3) / 1e9, 1)
            e["hbm_gbps_algorithmic"] = round(nbytes / (m * 1e-3) / 1e9, 1)
            e["roofline"] = roofline("mfma", f_method, m)
            if cfg["B"] <= 4:
                e["roofline"]["note"] = "launch-bound: the whole call is a few microseconds of launch overhead"
            ent["default"] = e
            torch.cuda.synchronize()
            dw_outputs[name] = yy.cpu().numpy().astype(np.float64)
            del yy
        configs[name] = ent

    # ---- variants, each against its own work
    def variant(fn, flops, nbytes, algorithm, bound="mfma", traffic_key=None):
        ms = time_calls(fn)
        m = float(np.median(ms))
        e = stats(ms)
        e["algorithm"] = algorithm
        e["gflops_own"] = round(flops / (m * 1e-3) / 1e9, 1)
        e["algorithmic_gflop_own"] = round(flops / 1e9, 3)
        e["roofline"] = roofline(bound, flops if bound == "mfma" else nbytes, m)
        if traffic_key:
            e["roofline"]["traffic"] = measured_traffic(traffic_key)
            e["trace_kernel_ms"] = trace_kernel_ms(traffic_key)
        return e

    f_conv, f_dw, f_tail = conv2d_flops(cc), dwsep_flops(dc), conv2d_flops(tc)
    b_conv, b_dw, b_tail = conv2d_bytes(cc), dwsep_bytes(dc), conv2d_bytes(tc)
    xt, wt, bt = gpu[TAIL]
    o1, o2 = torch.empty_like(out), torch.empty(tc["B"], device=dev)
    ws_det = torch.empty(fc.conv2d_det_workspace_bytes(cc["B"], cc["Cin"], cc["H"], cc["W"], cc["Cout"], cc["K"],
                                                       cc["pool"], fc.ALGO_DIRECT_MFMA) // 4, device=dev)
    variants = {
        "fconv2d_pool_sigmoid_sum_boxsum": variant(
            lambda: fc.conv2d_pool_sigmoid_sum(x, w, b, cc["pool"], out=o1, algo=fc.ALGO_BOXSUM),
            conv2d_boxsum_flops(cc), b_conv, "box-sum (FCONV_ALGO_BOXSUM, the default for this shape) on " + CONV
            + ": conv2d_pool_boxsum4_kernel (partial sums) + fixed-order reduction, HBM-bound", bound="hbm",
            traffic_key="conv2d_pool_boxsum4_kernel<2, true, 2, false>"),
        "fconv2d_pool_sigmoid_sum_det": variant(
            lambda: fc.conv2d_pool_sigmoid_sum_det(x, w, b, cc["pool"], out=o1, algo=fc.ALGO_DIRECT_MFMA,
                                                   workspace=ws_det),
            f_conv, b_conv, "direct MFMA with a caller-owned workspace for the partial sums (the default call takes it from the library pool) on " + CONV),
        "fconv2d_pool_sigmoid_sum_det_noalloc": variant(
            lambda: fc.conv2d_pool_sigmoid_sum_det_noalloc(x, w, b, cc["pool"], o1),
            conv2d_boxsum_flops(cc), b_conv, "allocation-free deterministic call (AUTO: box-sum partials in the "
            "library's fixed array + fixed-order reduction) on " + CONV, bound="hbm"),
        "fconv2d_pool_sigmoid_sum_ex_relu_maxpool": variant(
            lambda: fc.conv2d_pool_sigmoid_sum(x, w, b, cc["pool"], out=o1, algo=fc.ALGO_DIRECT_MFMA,
                                               pool_mode=fc.POOL_MAX, relu=True),
            f_conv, b_conv, "Conv2d -> ReLU -> MaxPool2d 4 (floor) -> sigmoid -> sum on " + CONV
            + ", per-conv-output MFMA kernel", traffic_key=ELEM_MAX),
        "fconv2d_pool_sigmoid_sum_k5s3_direct": variant(
            lambda: fc.conv2d_pool_sigmoid_sum(xt, wt, bt, tc["pool"], out=o2, algo=fc.ALGO_DIRECT_MFMA),
            f_tail, b_tail, "direct MFMA (pool folded into the contraction) on " + TAIL,
            traffic_key="conv2d_pool_mfma_kernel<fconv::DirectCfg<5, 3, 1, 3, 8, 1, 4, 12>, 2, false>"),
        "fconv2d_pool_sigmoid_sum_boxsum_k5s3": variant(
            lambda: fc.conv2d_pool_sigmoid_sum(xt, wt, bt, tc["pool"], out=o2, algo=fc.ALGO_BOXSUM),
            conv2d_boxsum_flops(tc), b_tail, "box-sum (the default for this shape) on " + TAIL
            + ", own FLOPs Cin*K*K per (co, pooled output)",
            traffic_key="conv2d_pool_boxsum_kernel<fconv::DirectCfg<5, 3, 1, 3, 8, 1, 4, 12>, 2, false>"),
        "fconv2d_pool_sigmoid_sum_ex_relu_maxpool_k5s3": variant(
            lambda: fc.conv2d_pool_sigmoid_sum(xt, wt, bt, tc["pool"], out=o2, algo=fc.ALGO_DIRECT_MFMA,
                                               pool_mode=fc.POOL_MAX, relu=True),
            f_tail, b_tail, "Conv2d k5 -> ReLU -> MaxPool2d 3 (floor) -> sigmoid -> sum on " + TAIL
            + ", per-conv-output MFMA kernel (K = 5, s = 3 instance)"),
    }
    # Cin 64: past the whole-tile LDS budget of the direct kernels, so DIRECT_MFMA runs the per-conv-output
    # kernel's channel-chunked tiling; AUTO runs box-sum (8-channel LDS chunks)
    wc = dict(B=16, Cin=64, H=384, W=384, Cout=64, K=3, pool=4)
    wide_host = fi.conv2d_inputs(wc["B"], wc["Cin"], wc["H"], wc["W"], wc["Cout"], wc["K"], seed=11)
    xw, ww, bw = (torch.from_numpy(a).to(dev) for a in wide_host)
    ow = {k: torch.empty(wc["B"], device=dev) for k in ("auto", "direct", "max")}
    wide_desc = "x[16,64,384,384] Conv2d 64->64 k3 -> "
    f_wide, b_wide = conv2d_flops(wc), conv2d_bytes(wc)
    bw_bound = "mfma" if conv2d_boxsum_flops(wc) / b_wide > PEAK_FP32_TFLOPS * 1e3 / PEAK_HBM_GBPS else "hbm"
    variants["fconv2d_pool_sigmoid_sum_cin64"] = variant(
        lambda: fc.conv2d_pool_sigmoid_sum(xw, ww, bw, wc["pool"], out=ow["auto"]),
        conv2d_boxsum_flops(wc), b_wide, "AUTO (box-sum, 8-channel LDS chunks) on " + wide_desc
        + "AvgPool2d 4 -> sigmoid -> sum, own FLOPs Cin*K*K per (co, pooled output)", bound=bw_bound)
    variants["fconv2d_pool_sigmoid_sum_cin64_direct"] = variant(
        lambda: fc.conv2d_pool_sigmoid_sum(xw, ww, bw, wc["pool"], out=ow["direct"], algo=fc.ALGO_DIRECT_MFMA),
        f_wide, b_wide, "direct MFMA, channel-chunked per-conv-output kernel (folded average pool) on "
        + wide_desc + "AvgPool2d 4 -> sigmoid -> sum")
    variants["fconv2d_pool_sigmoid_sum_ex_relu_maxpool_cin64"] = variant(
        lambda: fc.conv2d_pool_sigmoid_sum(xw, ww, bw, wc["pool"], out=ow["max"], algo=fc.ALGO_DIRECT_MFMA,
                                           pool_mode=fc.POOL_MAX, relu=True),
        f_wide, b_wide, "channel-chunked per-conv-output kernel on " + wide_desc
        + "ReLU -> MaxPool2d 4 (floor) -> sigmoid -> sum")
    torch.cuda.synchronize()
    wide_out = {k: v.cpu().numpy().astype(np.float64) for k, v in ow.items()}
    del xw, ww, bw, ow

    y_dense = torch.empty_like(y)
    variants["dwsep_conv1d_dense"] = variant(
        lambda: fc.dwsep_conv1d(xd, wdw, wpw, bpw, dc["pad"], out=y_dense, algo=fc.DWSEP_DENSE),
        dwsep_dense_flops(dc), b_dw, "dense-fused combined weight (FCONV_DWSEP_DENSE) on " + DW
        + ", own FLOPs C*K*O per step", traffic_key="dwsep_dense_kernel")
    torch.cuda.synchronize()
    variants["dwsep_conv1d_dense"]["matches_separable_within_tol"] = bool(
        ((y_dense - y).abs() <= 1e-4 + 1e-4 * y.abs()).all().item())

    # the conv1d generalisations at the dwsep_full scale: stride 2 (over twice the steps, so Tout is the
    # same), dilation 2 and 256 output channels, all on the tall tile; parity for these
    # forms is in tests/test_gpu_parity.py and tests/test_gpu_random_shapes.py
    def dw_gen(B, C, T, O, K, pad, stride, dil, seed):
        xg = torch.from_numpy(fi.dwsep_inputs(B, C, T, O, K, seed=seed)[0]).to(dev)
        To = (T + 2 * pad - dil * (K - 1) - 1) // stride + 1
        flops = 2 * B * To * C * (K + O)
        nbytes = 4 * (B * C * T + C * K + O * C + O + B * O * To)
        return xg, To, flops, nbytes
    x2, To2, f2, b2 = dw_gen(dc["B"], dc["C"], 2 * dc["T"], dc["O"], dc["K"], dc["pad"], 2, 1, seed=41)
    variants["dwsep_conv1d_stride2"] = variant(
        lambda: fc.dwsep_conv1d(x2, wdw, wpw, bpw, dc["pad"], out=y_dense, stride=2),
        f2, b2, f"stride 2 on x[{dc['B']},{dc['C']},{2 * dc['T']}] -> {dc['O']} channels (Tout {To2}), "
        "K 9, pad 4: the tall tile's stride-2 instance, own separable FLOPs")
    del x2
    xg = torch.from_numpy(fi.dwsep_inputs(dc["B"], dc["C"], dc["T"], dc["O"], dc["K"], seed=42)[0]).to(dev)
    f3 = 2 * dc["B"] * dc["T"] * dc["C"] * (dc["K"] + dc["O"])
    variants["dwsep_conv1d_dilation2"] = variant(
        lambda: fc.dwsep_conv1d(xg, wdw, wpw, bpw, 2 * dc["pad"], out=y_dense, dilation=2),
        f3, b_dw, f"dilation 2, pad 8 on {DW}: the tall tile's dilated instance, own separable FLOPs")
    del y_dense
    O4 = dc["O"] // 2
    y4 = torch.empty(dc["B"], O4, dc["T"], device=dev)
    w4, b4 = wpw[:O4].contiguous(), bpw[:O4].contiguous()
    f4 = 2 * dc["B"] * dc["T"] * dc["C"] * (dc["K"] + O4)
    b4b = 4 * (dc["B"] * dc["C"] * dc["T"] + dc["C"] * dc["K"] + O4 * dc["C"] + O4 + dc["B"] * O4 * dc["T"])
    variants["dwsep_conv1d_o256"] = variant(
        lambda: fc.dwsep_conv1d(xg, wdw, w4, b4, dc["pad"], out=y4),
        f4, b4b, f"x[{dc['B']},{dc['C']},{dc['T']}] -> {O4} channels, K 9, pad 4: the tall tile's 256-row "
        "instance, own separable FLOPs")
    del xg, y4, w4, b4

    # dwsep "cold": x and the weights (135 MB) fit in the 256 MB Infinity
    # Cache, so each timed call follows an overwrite of a 512 MB buffer; the
    # events bracket the call alone.
    flush = torch.empty((512 << 20) // 4, device=dev)
    cold = []
    for i in range(args.warmup + args.steps):
        flush.fill_(float(i))
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        dw_call()
        e1.record(stream)
        if i >= args.warmup:
            cold.append((e0, e1))
    torch.cuda.synchronize()
    ms_cold = np.array([e0.elapsed_time(e1) for e0, e1 in cold])
    del flush

    ceilings = measured_ceilings(torch, dev, stream)

    total_ms = start.elapsed_time(end)
    ms_step = total_ms / args.steps
    ms_conv = np.array([e[0].elapsed_time(e[1]) for e in ev])
    ms_dw = np.array([e[1].elapsed_time(e[2]) for e in ev])

    def kstats(ms, flops, nbytes):
        m = float(ms.mean())
        d = stats(ms)
        d.update({"gflops": round(flops / (m * 1e-3) / 1e9, 1),
                  "frac_fp32_peak": round(flops / (m * 1e-3) / (PEAK_FP32_TFLOPS * 1e12), 4),
                  "hbm_gbps_algorithmic": round(nbytes / (m * 1e-3) / 1e9, 1),
                  "algorithmic_gflop": round(flops / 1e9, 3), "algorithmic_bytes": nbytes})
        return d

    k_conv = kstats(ms_conv, f_conv, b_conv)
    k_conv["algorithm"] = ("FCONV_ALGO_DIRECT_MFMA: the direct convolution, s*s*Cin*K*K multiply-adds per "
                           "(co, pooled output); the entry point's default (AUTO) picks box-sum for this shape, "
                           "reported in configs.conv2d_full.default")
    k_dw = kstats(ms_dw, f_dw, b_dw)
    k_dw["algorithm"] = "FCONV_DWSEP_SEPARABLE (the default)"
    if "mfma_f32_16x16x4" in ceilings:
        ceil_tf = ceilings["mfma_f32_16x16x4"]["tflops"]
        for k, f in ((k_conv, f_conv), (k_dw, f_dw)):
            k["frac_of_measured_mfma_ceiling"] = round(f / (k["ms_mean"] * 1e-3) / 1e12 / ceil_tf, 4)
    k_conv["hbm_bytes_measured"] = measured_traffic(ELEM_AVG)
    k_conv["trace_kernel_ms"] = trace_kernel_ms(ELEM_AVG)
    k_dw["hbm_bytes_measured"] = measured_traffic(DW_TALL)
    k_dw["trace_kernel_ms"] = trace_kernel_ms(DW_TALL)
    k_dw["cold_ms_median"] = round(float(np.median(ms_cold)), 4)
    k_dw["cold_note"] = "each call after a 512 MB overwrite (inputs not in the 256 MB Infinity Cache)"
    # the box-sum call against the measured streaming-read rate too
    box = variants["fconv2d_pool_sigmoid_sum_boxsum"]
    box["trace_kernel_ms"] = trace_kernel_ms("conv2d_pool_boxsum4_kernel<2, true, 2, false>")
    if "hbm_read" in ceilings:
        box["roofline"]["frac_of_measured_read"] = round(box["roofline"]["achieved"] / ceilings["hbm_read"]["gbps"], 4)
        configs[CONV]["default"]["roofline"]["frac_of_measured_read"] = round(
            configs[CONV]["default"]["roofline"]["achieved"] / ceilings["hbm_read"]["gbps"], 4)
    achieved = f_conv / (k_conv["ms_mean"] * 1e-3) / 1e12

    result = {
        "metric": METRIC,
        "value": round((f_conv + f_dw) / (ms_step * 1e-3) / 1e9, 1),
        "unit": "GFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": ("synthetic: numpy PCG64 seeded with SeedSequence([seed, tensor id]), seed 0; x ~ N(0,1), "
                 "weights and biases ~ U(+-1/sqrt(fan_in)) (fconv_inputs.py); the same bytes feed the oracle"),
        "config": {
            "workload": f"{CONV} + {DW} (one call each per step)",
            CONV: "x[128,8,384,384] Conv2d 8->64 k3 -> AvgPool2d 4 -> sigmoid -> sum, direct convolution",
            DW: "x[32,256,4096] depthwise k9 pad4 -> pointwise 256->512 + bias",
            "parallelism": "single GPU",
        },
        "kernels": {"fconv2d_pool_sigmoid_sum": k_conv, "dwsep_conv1d": k_dw},
        "configs": configs,
        "variants": variants,
        "roofline": {
            "kernel": f"fconv2d_pool_sigmoid_sum, direct MFMA ({ELEM_AVG}) on " + CONV,
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": PEAK_FP32_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_FP32_TFLOPS, 4),
            "traffic": measured_traffic(ELEM_AVG),
            "traffic_unit": "bytes per launch (HBM, rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
            "frac_of_measured_ceiling": (round(achieved / ceilings["mfma_f32_16x16x4"]["tflops"], 4)
                                         if "mfma_f32_16x16x4" in ceilings else None),
        },
        "ceilings": ceilings,
        "timing": {"step": "one event triple per step around its two calls, on torch's current stream",
                   "configs_variants": f"median/p10/p90 over {args.reps} runs of {args.per_rep} back-to-back calls, "
                                       f"one event pair per run, after at least {args.call_warm_s} s of untimed "
                                       "runs of the same call"},
        "wall_s_timed_region": round(t_wall, 3),
        "settle": {"steps": settle_steps, "wall_s": round(t_settle, 3),
                   "note": "untimed whole steps before the warm-up, until the clocks leave their idle state"},
    }

    props = torch.cuda.get_device_properties(dev)
    result["device"] = {"name": props.name, "hip": getattr(torch.version, "hip", None),
                        "gcn_arch": getattr(props, "gcnArchName", None),
                        "compute_units": props.multi_processor_count}

    if not args.no_cpu_baseline:
        import oracle

        oracle.load()
        threads = oracle.oracle._threads(None)
        parity_ok = True
        t_base = {}
        for name, cfg in fi.WORKLOADS.items():
            arrs = host[name]
            t0 = time.perf_counter()
            if cfg["kind"] == "conv2d":
                want = oracle.conv2d_pool_sigmoid_sum(*arrs, cfg["pool"], nthreads=threads)
            else:
                want = oracle.dwsep_conv1d(*arrs, cfg["pad"], nthreads=threads)
            t = time.perf_counter() - t0
            t_base[name] = t
            par = {"oracle_s": round(t, 3), "oracle_threads": threads,
                   "checked": "every output of every batch item",
                   "rel_err_over": "outputs with |oracle| >= 1e-4"}
            if cfg["kind"] == "conv2d":
                for call_algo, key in ((0, "default"), (fc.ALGO_DIRECT_MFMA, "direct_mfma")):
                    if (name, call_algo) in conv_outputs:
                        r = err_over_tol(conv_outputs[(name, call_algo)], want)
                        par[f"{key}_max_err_over_tol"] = r
                        par[f"{key}_max_abs_err"], par[f"{key}_max_rel_err"] = abs_rel_err(
                            conv_outputs[(name, call_algo)], want)
                        parity_ok &= r <= 1.0
                if name == CONV:
                    r = err_over_tol(out.cpu().numpy(), want)   # the timed step's own results
                    par["step_max_err_over_tol"] = r
                    parity_ok &= r <= 1.0
            else:
                r = err_over_tol(dw_outputs[name], want)
                par["default_max_err_over_tol"] = r
                par["default_max_abs_err"], par["default_max_rel_err"] = abs_rel_err(dw_outputs[name], want)
                parity_ok &= r <= 1.0
                if name == DW:
                    r = err_over_tol(y.cpu().numpy(), want)
                    par["step_max_err_over_tol"] = r
                    parity_ok &= r <= 1.0
            par["oracle_gflops"] = round(configs[name]["algorithmic_gflop"] / t, 3)
            configs[name]["parity"] = par
        # the Cin-64 variants on their first and last batch items
        items = [0, wc["B"] - 1]
        t0 = time.perf_counter()
        want_avg = oracle.conv2d_pool_sigmoid_sum(*wide_host, wc["pool"], batch_idx=items, nthreads=threads)
        want_max = oracle.conv2d_pool_sigmoid_sum(*wide_host, wc["pool"], batch_idx=items, nthreads=threads,
                                                  pool_mode=oracle.POOL_MAX, relu=True)
        t_wide = time.perf_counter() - t0
        for key, got, want in (("fconv2d_pool_sigmoid_sum_cin64", "auto", want_avg),
                               ("fconv2d_pool_sigmoid_sum_cin64_direct", "direct", want_avg),
                               ("fconv2d_pool_sigmoid_sum_ex_relu_maxpool_cin64", "max", want_max)):
            r = err_over_tol(wide_out[got][items], want)
            variants[key]["parity"] = {"max_err_over_tol": r, "checked": f"batch items {items}, every output",
                                       "oracle_s_both_pools": round(t_wide, 3)}
            parity_ok &= r <= 1.0
        t_sample = t_base[CONV] + t_base[DW]
        result["cpu_baseline"] = {
            "value": round((f_conv + f_dw) / t_sample / 1e9, 3),
            "unit": "GFLOP/s",
            "cores": threads,
            "cpu_model": cpu_model(),
            "host_cpus": os.cpu_count(),
            "kind": "oracle",
            "sample": (f"literal float64 oracle on all {cc['B']} batch items of {CONV} ({t_base[CONV]:.1f} s) and "
                       f"all {dc['B']} of {DW} ({t_base[DW]:.1f} s), the step's inputs; every workload's oracle "
                       f"time is in configs.<name>.parity"),
        }
        result["parity_sample"] = {"ok": bool(parity_ok),
                                   "what": "every workload's default call (and direct call for the Conv2d ones) "
                                           "against the oracle on all batch items, and the Cin-64 variants on two, "
                                           "|err| / (1e-4 + 1e-4 |oracle|)"}
    else:
        result["cpu_baseline"] = None

    print(json.dumps(result), flush=True)
    # the oracle leg's parity check decides the exit status
    if result.get("parity_sample") and not result["parity_sample"]["ok"]:
        sys.exit(3)


if __name__ == "__main__":
    main()
