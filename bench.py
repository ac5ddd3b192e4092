"""Benchmark of the fused 3D conv / transposed-conv forward path on one MI355X.

One step = one pass of the whole hot path over one batch of synthetic input:
the five workloads back to back, each through its C-ABI entry point (inputs
resident in HBM, outputs and workspace preallocated):

  c1  conv3d_fwd              Conv3d 4->8 k3 p1 with bias, x[1,4,8,8,8] (launch-latency bound)
  c2  conv3d_fwd              Conv3d (3,3,1) kernel, depth-last x[16,3,256,256,10] -> [16,64,254,254,10]
  c3  conv_transpose3d_fwd    ConvTranspose3d 32->64 k3 s2 p1 d2, x[16,32,16,32,32] -> [16,64,33,65,65]
  c4  convT_bn_avgpool        ConvTranspose3d 3->16 k3 s2 p1 + BatchNorm3d (batch stats) + AvgPool3d(2) x2
  c5  conv_maxpool_lse_relu   Conv3d 32->64 k3 p1 + MaxPool3d(2) + logsumexp(dim=1) + ReLU, x[4,32,32,128,128]

value = effective TFLOP/s of the whole step = sum over workloads of 2*MAC / step time, where MAC is the
algorithmic work: the dense GEMM count for direct convs and the valid-tap count for transposed convs.

Prints one JSON line.  `--gpus N` with N > 1 exits: the library runs on one GPU.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

FP32_PEAK_TFLOPS = 157.3  # MI355X dense fp32 (MFMA and packed VALU)
HBM_PEAK_GBS = 8000.0     # MI355X HBM3E
BENCH_KEYS = ("c1", "c2", "c3", "c4", "c5")
# kernel that carries each workload (the roofline object names the dominant one)
CSRC = "transposed_convolution_epilogues_amd/csrc/"
KERNELS = {
    "c1": ("conv3d_k3_direct_kernel", [CSRC + "conv_direct.hip"]),
    "c2": ("conv_k1last_kernel", [CSRC + "conv_k1last.hip"]),
    "c3": ("conv333_store_kernel", [CSRC + "convT_sublattice.hip", CSRC + "conv333_mfma.h"]),
    "c4": ("swap_pool_kernel", [CSRC + "convT_bn_swap.hip"]),
    "c5": ("conv_pool_lse_mfma_kernel", [CSRC + "conv_pool_lse.hip", CSRC + "conv333_mfma.h"]),
}


def source_hash(paths):
    """SHA-256 prefix over a kernel's source files (traffic figures are only
    reported for the source they were measured on)."""
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def valid_pairs(L_in, k, s, p, d, L_out):
    return sum(1 for i in range(L_in) for kk in range(k) if 0 <= i * s - p + kk * d < L_out)


def work(wl, out_shape_conv):
    """(MAC_metric, algorithmic HBM bytes) of a workload."""
    N, cin = wl.x_shape[:2]
    cin_g = cin // wl.groups
    kvol = wl.kernel[0] * wl.kernel[1] * wl.kernel[2]
    O = out_shape_conv[2:]
    if wl.transposed:
        mac = N * wl.cout * cin_g
        for j in range(3):
            mac *= valid_pairs(wl.x_shape[2 + j], wl.kernel[j], wl.stride[j], wl.pad[j], wl.dilation[j], O[j])
    else:
        mac = N * wl.cout * O[0] * O[1] * O[2] * cin_g * kvol
    x_bytes = 4 * math.prod(wl.x_shape)
    w_bytes = 4 * math.prod(wl.weight_shape)
    return mac, x_bytes, w_bytes


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=4.0, help="target oracle seconds per workload sample")
    ap.add_argument("--only", default=None,
                    help="comma-separated subset of the workloads (or, with --widen, of its cases): profiling runs")
    ap.add_argument("--no-generic", action="store_true",
                    help="with --widen: skip the generic-kernel comparison (profiling runs)")
    ap.add_argument("--probe-mfma", action="store_true",
                    help="time the library's fp32 matrix-core throughput probe and print its TFLOP/s")
    ap.add_argument("--probe-valu", action="store_true",
                    help="time the probe with 0, 2, 4, 8 and 16 independent FMAs after every 4 MFMAs of a wave "
                         "(the cost of non-MFMA vector work beside the matrix cores) and print one JSON line")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run only a plain 1 GiB device-to-device copy (reference for HBM byte counters)")
    ap.add_argument("--widen", action="store_true",
                    help="instead of the step: time the work beyond the five configurations (general "
                         "transposed convs, eval-mode / running-statistics BatchNorm) against the generic kernels "
                         "and print one JSON line")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the library has no multi-GPU "
              "path: batch sharding across GPUs is a design note", file=sys.stderr)
        sys.exit(2)

    import torch

    if args.calibrate_copy:
        calibrate_copy(torch)
        return
    if args.probe_mfma:
        probe_mfma(torch)
        return
    if args.probe_valu:
        probe_valu(torch)
        return
    if args.widen:
        widen(torch, args)
        return

    from transposed_convolution_epilogues_amd import binding as B
    from transposed_convolution_epilogues_amd import workloads as W

    keys = [k for k in (args.only or ",".join(BENCH_KEYS)).split(",") if k]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    B.library()

    def g(a):
        return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    runs = {}
    for key in keys:
        wl = W.CONFIGS[key]
        inp = W.make_inputs(wl)
        x, w, b = g(inp.x), g(inp.w), g(inp.b)
        p = B.make_params(wl.kernel, wl.stride, wl.pad, wl.dilation, wl.output_pad, wl.groups)
        if wl.op == "conv3d":
            oshape = B.conv3d_out_dims(wl.x_shape, wl.cout, p)
            conv_shape = oshape
            y = torch.empty(oshape, device=dev)
            fn = (lambda x=x, w=w, b=b, y=y, wl=wl: B.conv3d_fwd(x, w, b, wl.stride, wl.pad, wl.dilation,
                                                                 wl.groups, out=y))
        elif wl.op == "conv_transpose3d":
            oshape = B.conv_transpose3d_out_dims(wl.x_shape, wl.cout, p)
            conv_shape = oshape
            y = torch.empty(oshape, device=dev)
            fn = (lambda x=x, w=w, b=b, y=y, wl=wl: B.conv_transpose3d_fwd(x, w, b, wl.stride, wl.pad, wl.dilation,
                                                                           wl.output_pad, wl.groups, out=y))
        elif wl.op == "convT_bn_avgpool":
            conv_shape = B.conv_transpose3d_out_dims(wl.x_shape, wl.cout, p)
            oshape = B.convT_bn_avgpool_out_dims(wl.x_shape, wl.cout, p, wl.pool)
            y = torch.empty(oshape, device=dev)
            ws = torch.empty(B.convT_bn_avgpool_workspace_bytes(wl.x_shape, wl.cout, p, wl.pool),
                             dtype=torch.uint8, device=dev)
            gm, bt = g(inp.gamma), g(inp.beta)
            fn = (lambda x=x, w=w, b=b, y=y, wl=wl, ws=ws, gm=gm, bt=bt:
                  B.convT_bn_avgpool(x, w, b, gm, bt, wl.eps, wl.pool, wl.stride, wl.pad, wl.dilation,
                                     wl.output_pad, wl.groups, out=y, workspace=ws))
        else:
            conv_shape = B.conv3d_out_dims(wl.x_shape, wl.cout, p)
            oshape = B.conv_maxpool_lse_relu_out_dims(wl.x_shape, wl.cout, p, wl.pool)
            y = torch.empty(oshape, device=dev)
            fn = (lambda x=x, w=w, b=b, y=y, wl=wl: B.conv_maxpool_lse_relu(x, w, b, wl.pool, wl.stride, wl.pad,
                                                                            wl.dilation, wl.groups, out=y))
        mac, xb, wb = work(wl, conv_shape)
        runs[key] = dict(wl=wl, fn=fn, mac=mac, bytes=xb + wb + 4 * math.prod(oshape), out_shape=oshape,
                         inp=inp, ev=[], y=y)
        print(f"[bench] {key}: {wl.description}; out {oshape}; MAC {mac:,}", file=sys.stderr, flush=True)

    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        for r in runs.values():
            r["fn"]()
    torch.cuda.synchronize()
    print(f"[bench] warmup done ({args.warmup} steps)", file=sys.stderr, flush=True)

    t0 = time.perf_counter()
    for _ in range(args.steps):
        for r in runs.values():
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            r["fn"]()
            e1.record(stream)
            r["ev"].append((e0, e1))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    print(f"[bench] timed {args.steps} steps: {ms_per_step:.3f} ms/step", file=sys.stderr, flush=True)

    per = {}
    total_flop = 0.0
    for key, r in runs.items():
        ms = [e0.elapsed_time(e1) for e0, e1 in r["ev"]]
        avg = float(np.mean(ms))
        flop = 2.0 * r["mac"]
        total_flop += flop
        p10, med, p90 = (float(v) for v in np.percentile(ms, [10, 50, 90]))
        per[key] = dict(op=r["wl"].op, ms_avg=round(avg, 5), ms_min=round(float(np.min(ms)), 5),
                        ms_median=round(med, 5), ms_p10=round(p10, 5), ms_p90=round(p90, 5),
                        tflops_median=round(flop / (med * 1e-3) / 1e12, 3),
                        tflops=round(flop / (avg * 1e-3) / 1e12, 3),
                        frac_fp32_peak=round(flop / (avg * 1e-3) / 1e12 / FP32_PEAK_TFLOPS, 4),
                        hbm_gbs=round(r["bytes"] / (avg * 1e-3) / 1e9, 1),
                        frac_hbm_peak=round(r["bytes"] / (avg * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                        mac=r["mac"], algo_bytes=r["bytes"], out_shape=list(r["out_shape"]))
    value = total_flop / (ms_per_step * 1e-3) / 1e12
    # outside the timed region: each workload alone, back to back (warm: its
    # inputs may sit in L2 and the 256 MB MALL), and after a 512 MB write that
    # evicts both (cold)
    for key, (warm, cold) in warm_cold(torch, runs, stream).items():
        per[key].update(ms_warm_median=round(warm, 5), ms_cold_median=round(cold, 5))

    # roofline object for the dominant kernel (largest average duration)
    dom = max(per, key=lambda k: per[k]["ms_avg"])
    kname, ksrcs = KERNELS[dom]
    bound = "mfma" if dom in ("c3", "c5") else ("hbm" if dom == "c2" else "alu")
    if bound == "hbm":
        achieved = per[dom]["algo_bytes"] / (per[dom]["ms_avg"] * 1e-3) / 1e9
        peak, unit = HBM_PEAK_GBS, "GB/s"
    else:
        achieved = 2.0 * per[dom]["mac"] / (per[dom]["ms_avg"] * 1e-3) / 1e12
        peak, unit = (FP32_PEAK_TFLOPS if bound == "mfma" else FP32_PEAK_TFLOPS / 2), "TFLOP/s"
    traffic = None
    tfile = os.path.join(ROOT, "profiles", f"{kname}_{dom}_traffic.json")
    if os.path.exists(tfile):
        with open(tfile) as f:
            tr = json.load(f)
        if tr.get("source_sha256_16") == source_hash(ksrcs):
            traffic = tr.get("hbm_bytes_per_launch")
    roofline = dict(kernel=kname, workload=dom, bound=bound, achieved=round(achieved, 3), peak=peak, unit=unit,
                    frac=round(achieved / peak, 4), traffic=traffic)

    hw = hardware(torch)
    cpu = None
    if not args.no_cpu_baseline:
        cpu, errs = cpu_baseline(runs, args.cpu_seconds)
        for key, e in errs.items():
            per[key].update(e)
            per[key]["oracle_cores"] = cpu["cores"]

    line = {
        "metric": "effective TFLOP/s (2*MACs/time) and % of MI355X fp32 peak, per config",
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded U[-1,1] inputs, PyTorch-default uniform weights)",
        "config": {
            "workload": "fused 3D conv suite, one pass of c1+c2+c3+c4+c5 at full size: " +
                        "; ".join(f"{k}: {runs[k]['wl'].description}" for k in runs),
            "per_config": per,
            "frac_fp32_peak_step": round(value / FP32_PEAK_TFLOPS, 4),
        },
        "roofline": roofline,
        "cpu_baseline": cpu,
        "hw": hw,
    }
    print(json.dumps(line), flush=True)


def measure_probe(torch, reps=10):
    """Achievable fp32 MFMA throughput on this GPU: back-to-back independent
    v_mfma_f32_32x32x2f32 chains, two waves per SIMD on every CU."""
    from transposed_convolution_epilogues_amd import binding as B
    out = torch.empty(2048 * 256, dtype=torch.float32, device="cuda")
    iters = 2000
    for _ in range(3):
        flop = B.probe_mfma_f32(iters, out)
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        B.probe_mfma_f32(iters, out)
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    ts.sort()
    med = ts[len(ts) // 2]
    return {"probe": "mfma_f32_32x32x2", "flop": flop, "ms_median": round(med, 4),
            "tflops": round(flop / (med * 1e-3) / 1e12, 2), "peak": FP32_PEAK_TFLOPS,
            "frac_of_peak": round(flop / (med * 1e-3) / 1e12 / FP32_PEAK_TFLOPS, 4)}


def probe_mfma(torch):
    print(json.dumps(measure_probe(torch)), flush=True)


def probe_valu(torch, reps=7):
    """MFMA throughput of the probe with v FMAs after every 4 MFMAs of a wave."""
    from transposed_convolution_epilogues_amd import binding as B
    out = torch.empty(2048 * 256, dtype=torch.float32, device="cuda")
    iters = 2000
    rows = []
    for v in (0, 2, 4, 8, 16):
        call = (lambda: B.probe_mfma_f32(iters, out)) if v == 0 else (lambda: B.probe_mfma_valu_f32(iters, v, out))
        for _ in range(2):
            flop = call()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            call()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        ts.sort()
        med = ts[len(ts) // 2]
        rows.append({"valu_per_mfma": v / 4, "ms_median": round(med, 4),
                     "mfma_tflops": round(flop / (med * 1e-3) / 1e12, 2)})
    print(json.dumps({"probe": "mfma_f32_32x32x2 with independent v_fma_f32 beside it", "rows": rows}), flush=True)


def gpu_clocks():
    """Current shader clock (MHz) from the driver's sysfs table of sclk levels
    (the active level is marked '*'), or None.  A file read: no other program
    is started from this process, which has initialised the GPU."""
    import glob
    import re
    for path in sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk")):
        try:
            with open(path) as f:
                for line in f:
                    if "*" in line:
                        m = re.search(r"(\d+)\s*Mhz", line, re.I)
                        if m:
                            return int(m.group(1))
        except OSError:
            continue
    return None


def hardware(torch):
    """What the line's peaks are checked against: the device, its clocks and
    the measured matrix-core throughput, taken after the timed steps."""
    prop = torch.cuda.get_device_properties(0)
    hw = {"device": prop.name, "gcn_arch": getattr(prop, "gcnArchName", None),
          "compute_units": prop.multi_processor_count,
          "max_clock_mhz": None, "sclk_mhz_after_run": gpu_clocks()}
    try:
        from transposed_convolution_epilogues_amd import binding as B  # noqa: F401
        import ctypes
        hip = ctypes.CDLL("libamdhip64.so")
        rate = ctypes.c_int(0)
        # hipDeviceAttributeClockRate = 5 (kHz)
        if hip.hipDeviceGetAttribute(ctypes.byref(rate), 5, 0) == 0:
            hw["max_clock_mhz"] = rate.value // 1000
    except OSError:
        pass
    hw["mfma_probe"] = measure_probe(torch, reps=5)
    return hw


def calibrate_copy(torch):
    """A plain copy of known size: each launch reads and writes exactly 1 GiB.
    Its FETCH_SIZE / WRITE_SIZE counter readings give the scale that turns the
    counters into HBM bytes for the library's kernels."""
    nbytes = 1 << 30
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 5
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    print(json.dumps({"copy_bytes_read": nbytes, "copy_bytes_written": nbytes, "ms": round(ms, 4),
                      "gbs_read_plus_write": round(2 * nbytes / (ms * 1e-3) / 1e9, 1)}), flush=True)


def widen(torch, args):
    """Work beyond the five configurations, each timed through its automatic
    kernel and through the generic kernels for comparison:
      - transposed convs on the shared-halo phase kernel and on the
        one-phase-per-workgroup kernel, the c3 module through both general
        paths instead of its sub-lattice kernel, and both through the
        LDS-scatter algorithm;
      - the c4 module with BatchNorm in eval mode (running statistics), in
        training mode with the running-statistics update, and through its
        second algorithm (the output-phase classes on the matrix cores)."""
    from transposed_convolution_epilogues_amd import binding as B
    from transposed_convolution_epilogues_amd import workloads as W

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    B.library()
    c4 = W.CONFIGS["c4"]
    cases = ([(k, wl, 0, "convT") for k, wl in W.WIDEN.items()] +
             [(k + "_per_phase", wl, 6, "convT") for k, wl in W.WIDEN.items()] +
             [("c3_phase", W.CONFIGS["c3"], 2, "convT"), ("c3_per_phase", W.CONFIGS["c3"], 6, "convT")] +
             [("t1_scatter", W.WIDEN["t1"], 4, "convT"), ("c3_scatter", W.CONFIGS["c3"], 4, "convT")] +
             [("c4_eval", c4, 0, "bn_eval"), ("c4_train_running", c4, 0, "bn_running"),
              ("c4_phase_classes", c4, 3, "bn_second")])
    if args.only:
        sel = set(args.only.split(","))
        cases = [c for c in cases if c[0] in sel]
    out = {}
    for key, wl, variant, kind in cases:
        inp = W.make_inputs(wl)
        t = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(dev)
        x, w, b = t(inp.x), t(inp.w), t(inp.b)
        p = B.make_params(wl.kernel, wl.stride, wl.pad, wl.dilation, wl.output_pad, wl.groups)
        conv_shape = B.conv_transpose3d_out_dims(wl.x_shape, wl.cout, p)
        mac, xb, wb = work(wl, conv_shape)
        kw = dict(stride=wl.stride, pad=wl.pad, dilation=wl.dilation, output_pad=wl.output_pad, groups=wl.groups)
        if kind == "convT":
            y = torch.empty(conv_shape, device=dev)
            fn = lambda: B.conv_transpose3d_fwd(x, w, b, out=y, **kw)
            algo = lambda: B.conv_transpose3d_algo(wl.x_shape, wl.cout, p)
        else:
            y = torch.empty(B.convT_bn_avgpool_out_dims(wl.x_shape, wl.cout, p, wl.pool), device=dev)
            gm, bt = t(inp.gamma), t(inp.beta)
            rm0, rv0 = W.make_running_stats(wl.cout, 5)
            rm, rv = t(rm0), t(rv0)
            ws = torch.empty(B.convT_bn_avgpool_workspace_bytes(wl.x_shape, wl.cout, p, wl.pool), dtype=torch.uint8,
                             device=dev)
            if kind == "bn_second":  # the module's second algorithm, batch statistics only
                fn = lambda: B.convT_bn_avgpool(x, w, b, gm, bt, wl.eps, wl.pool, out=y, workspace=ws, **kw)
            else:
                train = kind == "bn_running"
                fn = lambda: B.convT_bn_avgpool(x, w, b, gm, bt, wl.eps, wl.pool, out=y, workspace=ws,
                                                training=train, running_mean=rm, running_var=rv, **kw)
            algo = lambda: B.convT_bn_avgpool_algo(wl.x_shape, wl.cout, p, wl.pool)
        nbytes = xb + wb + 4 * y.numel()
        row = dict(workload=wl.description + {"convT": "", "bn_eval": "; BN in eval mode",
                                              "bn_running": "; training mode + running-statistics update",
                                              "bn_second": "; output-phase classes on the matrix cores"}[kind],
                   mac=mac, algo_bytes=nbytes)
        legs = (("fast", variant, args.steps),) + (() if args.no_generic else (("generic", 1, 3),))
        for label, v, reps in legs:
            old = B.set_variant(v)
            try:
                row[label + "_algo"] = algo() if v != 1 else "generic"
                for _ in range(2):
                    fn()
                torch.cuda.synchronize()
                ms = []
                stream = torch.cuda.current_stream()
                for _ in range(reps):
                    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    e0.record(stream)
                    fn()
                    e1.record(stream)
                    ms.append((e0, e1))
                torch.cuda.synchronize()
                tm = float(np.median([a.elapsed_time(c) for a, c in ms]))
            finally:
                B.set_variant(old)
            row[label + "_ms_median"] = round(tm, 5)
            row[label + "_tflops"] = round(2.0 * mac / (tm * 1e-3) / 1e12, 3)
        row["frac_fp32_peak"] = round(row["fast_tflops"] / FP32_PEAK_TFLOPS, 4)
        row["hbm_gbs"] = round(nbytes / (row["fast_ms_median"] * 1e-3) / 1e9, 1)
        row["frac_hbm_peak"] = round(row["hbm_gbs"] / HBM_PEAK_GBS, 4)
        if "generic_ms_median" in row:
            row["speedup_vs_generic"] = round(row["generic_ms_median"] / row["fast_ms_median"], 2)
        out[key] = row
        print(f"[bench --widen] {key}: {row}", file=sys.stderr, flush=True)
        del x, w, b, y
    print(json.dumps({"metric": "effective TFLOP/s (2*MACs/time; valid-tap MACs for transposed convs), work beyond "
                                "the five configurations", "unit": "TFLOP/s", "dtype": "f32", "data": "synthetic",
                      "steps": args.steps, "widen": out}), flush=True)


def warm_cold(torch, runs, stream, calls=20):
    """Median event-timed duration (ms) of each workload called on its own:
    back to back (warm), and each call after a 512 MB scratch write (cold)."""
    flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda:0")
    out = {}
    for key, r in runs.items():
        res = []
        for cold in (False, True):
            ev = []
            for _ in range(calls):
                if cold:
                    flush.fill_(1)
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                r["fn"]()
                e1.record(stream)
                ev.append((e0, e1))
            torch.cuda.synchronize()
            res.append(float(np.median([a.elapsed_time(b) for a, b in ev])))
        out[key] = tuple(res)
    del flush
    return out


def errors(got, ref):
    """max |gpu - oracle|, the max relative error over outputs with |oracle| >= 1e-3,
    and the largest error as a fraction of the parity bar 1e-4 + 1e-4 |oracle|."""
    got = np.asarray(got, np.float64).ravel()
    ref = np.asarray(ref, np.float64).ravel()
    err = np.abs(got - ref)
    big = np.abs(ref) >= 1e-3
    return {"max_abs_err": float(err.max()),
            "max_rel_err": float((err[big] / np.abs(ref[big])).max()) if big.any() else 0.0,
            "err_over_tol": float((err / (1e-4 + 1e-4 * np.abs(ref))).max()),
            "checked": int(err.size)}


def cpu_baseline(runs, seconds_per_workload):
    """The CPU oracle, timed on a bounded sample of each workload and scaled to the
    whole workload; reported in the same effective TFLOP/s as the GPU value.  The
    same oracle outputs are compared with the GPU's outputs of the last timed
    step (errors per workload)."""
    import oracle as O

    rng = np.random.default_rng(0)
    total_flop = 0.0
    total_s = 0.0
    parts = []
    errs = {}
    for key, r in runs.items():
        wl, inp = r["wl"], r["inp"]
        kw = dict(stride=wl.stride, pad=wl.pad, dilation=wl.dilation, groups=wl.groups)
        full_units = math.prod(r["out_shape"])
        y = r["y"].detach().cpu().numpy()
        if wl.op == "convT_bn_avgpool" or full_units <= 65536:
            # the whole module (BatchNorm needs whole-batch statistics; c1 is tiny)
            t0 = time.perf_counter()
            ref = O.run_workload(wl, inp)
            dt = time.perf_counter() - t0
            ref = ref[0] if isinstance(ref, tuple) else ref
            errs[key] = errors(y, ref)
            frac = 1.0
            desc = f"{key}: whole workload"
        else:
            n = 256
            while True:
                flat = rng.integers(0, full_units, n)
                t0 = time.perf_counter()
                if wl.op == "conv3d":
                    ref = O.conv3d_at(inp.x, inp.w, flat, inp.b, **kw)
                elif wl.op == "conv_transpose3d":
                    ref = O.conv_transpose3d_at(inp.x, inp.w, flat, inp.b, output_pad=wl.output_pad, **kw)
                else:
                    ref = O.conv_maxpool_lse_relu_at(inp.x, inp.w, inp.b, flat, wl.pool, **kw)
                dt = time.perf_counter() - t0
                if dt > seconds_per_workload / 4 or n >= full_units:
                    break
                n *= 4
            errs[key] = errors(y.reshape(-1)[flat], ref)
            frac = n / full_units
            desc = f"{key}: {n} random outputs of {full_units}"
        t_full = dt / frac
        errs[key]["oracle_s"] = round(t_full, 3)
        errs[key]["oracle_s_scope"] = "measured" if frac == 1.0 else f"scaled from {n} sampled outputs"
        total_s += t_full
        total_flop += 2.0 * r["mac"]
        parts.append(f"{desc} in {dt:.2f}s")
        print(f"[bench] cpu oracle {desc}: {dt:.2f}s -> {t_full:.1f}s for the whole workload; {errs[key]}",
              file=sys.stderr, flush=True)
    cpu = {"value": round(total_flop / total_s / 1e12, 6), "unit": "TFLOP/s", "cores": O.num_threads(),
           "kind": "oracle",
           "sample": "plain-loop float64 oracle timed on bounded samples, scaled to the whole step: " +
                     "; ".join(parts)}
    return cpu, errs


if __name__ == "__main__":
    main()
