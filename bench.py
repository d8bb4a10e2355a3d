#!/usr/bin/env python3
"""Benchmark of the fused fp32 convolution hot path on one MI355X.

One step = one call of each entry point on its full-size workload, in this order:
  conv3d_div_maxpool_gap_bias_sum  x [128,8,16,64,64]      -> out [128]
  conv3d_mish_tanh                 x [16,32,32,64,64]      -> y [16,64,30,62,62]
  dwsep_conv2d                     x [16,64,512,512]       -> y [16,128,512,512]
  dwsep_conv2d (odd, biased)       x [8,96,333,517]        -> y [8,192,333,517]
Inputs are seeded synthetic tensors already resident in HBM when timing starts.
`value` is the step's convolution work (2 x multiply-adds) per second, in TFLOP/s, over
`--steps` timed steps; each launch in them is also timed with HIP events on its stream (the
`roofline` object uses those averages).  After the timed steps every workload is launched
alone `--reps` times with the caches flushed before each launch (a 512 MiB write, then a
512 MiB read of another buffer: the headline per-workload time is the median of these) and
`--reps` times back to back (the warm median); the tiny configuration [1,4,8,16,16] is timed
the same way over `--tiny-reps` launches (reported, not graded).  Each workload's record gives
its rates against the fp32 matrix peak (matrix-core FLOP only: the depthwise step of the
separable layers runs on the vector ALUs and is listed apart) and against HBM, and the roof
it is graded on.  The CPU baseline runs the fp64 oracle over the same workloads, with the
wall time of each.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time
from pathlib import Path

import numpy as np

ROOT = Path(__file__).resolve().parent
sys.path.insert(0, str(ROOT))

PEAK_FP32_TFLOPS = 157.3   # MI355X dense fp32 matrix peak
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E
BENCH_WORKLOADS = (2, 3, 4, 5)


def _olen(n, k, s=1, p=0, d=1):
    return (n + 2 * p - d * (k - 1) - 1) // s + 1


def out_dims(w):
    """Output spatial sizes of the convolution(s) of a workload."""
    d, p = w.dims, w.params
    if w.op.startswith("dwsep_conv2d"):
        args = (p["K"], p["stride"], p["pad"], p["dilation"])
        return _olen(d["H"], *args), _olen(d["W"], *args)
    s, pad = p.get("stride", 1), p.get("pad", 0)
    return tuple(_olen(d[a], p["k"], s, pad) for a in ("D", "H", "W"))


def work(w):
    """Algorithmic multiply-adds and bytes (inputs + weights + outputs, each once)."""
    d, p = w.dims, w.params
    if w.op.startswith("conv3d_mish_tanh"):
        k = p["k"]
        od, oh, ow = out_dims(w)
        outs = d["N"] * d["O"] * od * oh * ow
        macs = outs * d["C"] * k ** 3
        nbytes = 4 * (d["N"] * d["C"] * d["D"] * d["H"] * d["W"] + d["O"] * d["C"] * k ** 3
                      + d["O"] + outs)
    elif w.op.startswith("conv3d_div_maxpool"):
        k, pool = p["k"], p["pool"]
        od, oh, ow = out_dims(w)
        pooled = [(s - pool) // pool + 1 for s in (od, oh, ow)]
        # only the conv outputs some window reads: floor-mode pooling never reads the rest
        # (none for a 2x2x2 pool on even sizes)
        used = d["N"] * d["O"] * pool ** 3 * pooled[0] * pooled[1] * pooled[2]
        macs = used * d["C"] * k ** 3
        nbytes = 4 * (d["N"] * d["C"] * d["D"] * d["H"] * d["W"] + d["O"] * d["C"] * k ** 3)
        if w.op == "conv3d_div_maxpool":
            nbytes += 4 * (d["O"] + d["N"] * d["O"] * pooled[0] * pooled[1] * pooled[2])
        else:
            nbytes += 4 * (2 * d["O"] + d["N"])
    else:
        K = p["K"]
        ho, wo = out_dims(w)
        pix_in, pix_out = d["N"] * d["H"] * d["W"], d["N"] * ho * wo
        macs = pix_out * d["C"] * K * K + pix_out * d["O"] * d["C"]
        nbytes = 4 * (pix_in * d["C"] + d["C"] * K * K + d["O"] * d["C"] + pix_out * d["O"]
                      + (d["C"] + d["O"] if p["bias"] else 0))
    return macs, nbytes


def gemm_macs(w):
    """The multiply-adds that run as a matrix contraction on the fp32 matrix cores: the whole
    Conv3d, but only the pointwise step of a depthwise-separable layer (its depthwise step
    runs on the vector ALUs)."""
    macs, _ = work(w)
    if w.op.startswith("dwsep_conv2d"):
        K = w.params["K"]
        ho, wo = out_dims(w)
        macs -= w.dims["N"] * ho * wo * w.dims["C"] * K * K
    return macs


def graded_bound(w):
    """The roof a layer is judged against: HBM for the depthwise-separable layers, the fp32
    matrix cores for the Conv3d layers."""
    return "hbm" if w.op.startswith("dwsep_conv2d") else "mfma"


def kernel_name(w):
    """The kernel a workload's entry point launches (the launchers' dispatch rules)."""
    p = w.params
    if w.op.startswith("conv3d_mish_tanh"):
        if p["k"] == 3 and p["stride"] == 1 and p["pad"] <= 2:
            return "conv3d_mish_tanh_kernel" if w.op == "conv3d_mish_tanh" else "conv3d_split_kernel"
        if p["k"] in (3, 5, 7) and p["stride"] in (1, 2):
            return "conv3d_staged_kernel"
        return "conv3d_mish_tanh_generic_kernel"
    if w.op.startswith("conv3d_div_maxpool"):
        if p["k"] == 3 and p["pool"] == 2:
            return ("conv3d_pool_split_kernel" if w.op.endswith("split_bf16")
                    else "conv3d_pool_sum_kernel")
        if p["k"] in (1, 3, 5) and p["pool"] in (2, 3, 4):
            return "conv3d_pool_staged_kernel"
        return "conv3d_pool_sum_generic_kernel"
    tuned = p["K"] == 3 and p["stride"] == 1 and p["dilation"] == 1 and p["pad"] <= 2
    if w.op == "dwsep_conv2d_split_bf16" and tuned:
        return "dwsep_split_kernel"
    return "dwsep_persistent_kernel" if tuned else "dwsep_staged_kernel"


def kernel_source_sha():
    """Source hash the loaded libconvfuse.so was compiled from (stamped in by the build)."""
    import implicit_gemm_convolution_conv3d_amd as cf
    return cf.build_id()


def load_traffic(kernel_name):
    """HBM bytes per launch from the committed rocprofv3 counter summary, only if it was
    taken on the current kernel sources."""
    f = ROOT / "profiles" / "traffic.json"
    if not f.exists():
        return None
    try:
        data = json.loads(f.read_text())
    except ValueError:
        return None
    ent = data.get(kernel_name)
    if not ent or ent.get("kernel_source_sha") != kernel_source_sha():
        return None
    return ent.get("hbm_bytes_per_launch")


# kernel name prefix (as rocprofv3 prints it) -> workload it serves in the bench step
KERNEL_PREFIX = {"conv3d_pool_sum_kernel": "conv3d_div_maxpool_gap_bias_sum",
                 "conv3d_mish_tanh_kernel": "conv3d_mish_tanh",
                 "dwsep_persistent_kernel<8,": "dwsep_conv2d_512",
                 "dwsep_persistent_kernel<12,": "dwsep_conv2d_333x517_bias"}


def summarize_traffic(fetch_csv, write_csv, calib_mib):
    """HBM bytes per launch of each kernel from rocprofv3 FETCH_SIZE / WRITE_SIZE (KiB per
    dispatch), each scaled by what the same counter reads for a device multiply over calib_mib MiB
    (the multiply reads and writes exactly that many bytes)."""
    import csv

    def per_kernel(path, counter):
        acc = {}
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            acc.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        return {k: sum(v) / len(v) for k, v in acc.items()}

    fetch, write = per_kernel(fetch_csv, "FETCH_SIZE"), per_kernel(write_csv, "WRITE_SIZE")
    calib = calib_mib * (1 << 20)
    # the calibration kernel is torch's elementwise multiply (reads and writes calib bytes)
    copy_f = max((v for k, v in fetch.items() if "MulFunctor" in k), default=None)
    copy_w = max((v for k, v in write.items() if "MulFunctor" in k), default=None)
    if not copy_f or not copy_w:
        raise SystemExit("no calibration multiply kernel found in the counter files")
    fscale, wscale = calib / (copy_f * 1024), calib / (copy_w * 1024)
    out = {"_about": "HBM bytes per launch = FETCH_SIZE*1024*fetch_scale + WRITE_SIZE*1024*"
                     "write_scale; scales from a %d MiB device multiply (read + write)" % calib_mib,
           "fetch_scale": round(fscale, 4), "write_scale": round(wscale, 4)}
    sha = kernel_source_sha()
    for kname, f in fetch.items():
        for pre, wl_name in KERNEL_PREFIX.items():
            if pre in kname and kname in write:
                fb, wb = f * 1024 * fscale, write[kname] * 1024 * wscale
                out[wl_name] = {"kernel": kname[:120], "kernel_source_sha": sha,
                                "fetch_bytes": round(fb), "write_bytes": round(wb),
                                "hbm_bytes_per_launch": round(fb + wb)}
    dst = ROOT / "profiles" / "traffic.json"
    dst.write_text(json.dumps(out, indent=1) + "\n")
    print(json.dumps(out, indent=1))


def run_op(cf, w, t, out):
    p = w.params
    if w.op.startswith("conv3d_mish_tanh"):
        fn = cf.conv3d_mish_tanh if w.op == "conv3d_mish_tanh" else cf.conv3d_mish_tanh_split_bf16
        fn(t["x"], t["w"], t["b"], p["stride"], p["pad"], out=out)
    elif w.op.startswith("conv3d_div_maxpool_gap_bias_sum"):
        fn = (cf.conv3d_div_maxpool_gap_bias_sum if w.op == "conv3d_div_maxpool_gap_bias_sum"
              else cf.conv3d_div_maxpool_gap_bias_sum_split_bf16)
        fn(t["x"], t["w"], t["conv_b"], p["divisor"], p["pool"], t["bias"], out=out)
    elif w.op == "conv3d_div_maxpool":
        cf.conv3d_div_maxpool(t["x"], t["w"], t["conv_b"], p["divisor"], p["pool"], out=out)
    else:
        fn = cf.dwsep_conv2d if w.op == "dwsep_conv2d" else cf.dwsep_conv2d_split_bf16
        fn(t["x"], t["dw_w"], t["dw_b"], t["pw_w"], t["pw_b"], p["stride"], p["pad"],
           p["dilation"], out=out)


def out_shape(w):
    d = w.dims
    if w.op.startswith("conv3d_mish_tanh"):
        return (d["N"], d["O"]) + out_dims(w)
    if w.op.startswith("conv3d_div_maxpool_gap_bias_sum"):
        return (d["N"],)
    if w.op == "conv3d_div_maxpool":
        pool = w.params["pool"]
        return (d["N"], d["O"]) + tuple((s - pool) // pool + 1 for s in out_dims(w))
    return (d["N"], d["O"]) + out_dims(w)


def cpu_baseline(workloads, frac_batch):
    """The fp64 oracle, untouched, on the first batch items of each workload.  Input
    generation is outside the timed region.  Returns (TFLOP/s over all of them, threads,
    description, per-workload {wall_s, gflop, gflops, batch_items})."""
    import oracle
    total_macs, secs, parts, per = 0, 0.0, [], {}
    for w in workloads:
        d, p = w.dims, w.params
        nb = max(1, int(round(d["N"] * frac_batch)))
        inp = w.inputs()
        x = np.ascontiguousarray(inp["x"][:nb])
        macs, _ = work(w)
        t0 = time.perf_counter()
        if w.op == "conv3d_mish_tanh":
            oracle.conv3d_mish_tanh(x, inp["w"], inp["b"], p["stride"], p["pad"])
        elif w.op == "conv3d_div_maxpool_gap_bias_sum":
            oracle.conv3d_div_maxpool_gap_bias_sum(x, inp["w"], inp["conv_b"], p["divisor"],
                                                   p["pool"], inp["bias"])
        elif w.op == "conv3d_div_maxpool":
            oracle.conv3d_div_maxpool(x, inp["w"], inp["conv_b"], p["divisor"], p["pool"])
        else:
            oracle.dwsep_conv2d(x, inp["dw_w"], inp["dw_b"], inp["pw_w"], inp["pw_b"],
                                p["stride"], p["pad"], p["dilation"])
        dt = time.perf_counter() - t0
        secs += dt
        m = macs * nb // d["N"]
        total_macs += m
        per[w.name] = {"wall_s": round(dt, 3), "gflop": round(2 * m / 1e9, 3),
                       "gflops": round(2 * m / dt / 1e9, 2),
                       "batch_items": "%d of %d" % (nb, d["N"])}
        parts.append("%s batch items 0..%d of %d" % (w.name, nb - 1, d["N"]))
        del inp, x
    desc = "; ".join(parts) + " (%.1f s of fp64 naive loops)" % secs
    return 2 * total_macs / secs / 1e12, oracle.threads(), desc, per


def ceilings(cf, reps):
    """Practical ceilings on this GPU: the fp32 MFMA issue rate (convfuse_measure_mfma: 8
    workgroups of 4 waves per CU, 16 independent accumulators per wave, no memory traffic)
    and the HBM rate of torch's copy and fill over 1 GiB.  Median of `reps` launches each,
    HIP events on the launch stream."""
    import torch
    stream = torch.cuda.current_stream()

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        ms = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            e1.synchronize()
            ms.append(e0.elapsed_time(e1))
        return float(np.median(ms))

    out = torch.zeros(1, device="cuda:0")
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    wgs, iters = 8 * cus, 2048
    t_mfma = timed(lambda: cf.measure_mfma(iters, wgs, out))
    assert out.item() == iters * 2.0 ** -14  # the loop ran every MFMA
    mfma_tf = wgs * 4 * iters * 16 * 2048 / (t_mfma * 1e-3) / 1e12
    n = 1 << 28
    src = torch.ones(n, device="cuda:0")
    dst = torch.empty_like(src)
    t_copy = timed(lambda: dst.copy_(src))
    t_fill = timed(lambda: dst.fill_(2.0))
    res = {
        "fp32_mfma_tflops": round(mfma_tf, 1),
        "fp32_mfma_frac_of_spec": round(mfma_tf / PEAK_FP32_TFLOPS, 4),
        "copy_gbs": round(8 * n / (t_copy * 1e-3) / 1e9, 1),
        "fill_gbs": round(4 * n / (t_fill * 1e-3) / 1e9, 1),
        "cus": cus,
    }
    del src, dst
    torch.cuda.empty_cache()
    return res


def host_info():
    """The host the CPU baseline ran on: the full model string and identifiers from
    /proc/cpuinfo, the cores this process may use, and the OpenMP thread setting."""
    info = {"cpu_model": "unknown"}
    try:
        for line in open("/proc/cpuinfo"):
            key, _, val = line.partition(":")
            key, val = key.strip(), val.strip()
            if key == "model name" and info["cpu_model"] == "unknown":
                info["cpu_model"] = val
            elif key in ("vendor_id", "cpu family", "model", "stepping") and key not in info:
                info[key.replace(" ", "_")] = val
    except OSError:
        pass
    info["nproc"] = len(os.sched_getaffinity(0))
    info["os_cpu_count"] = os.cpu_count()
    info["OMP_NUM_THREADS"] = os.environ.get("OMP_NUM_THREADS")
    return info


def ablation(cf, wls, steps, warmup):
    """Fused entry point against the unfused path built from the same kernels (conv writing
    its output, then the epilogue or reduction as separate kernels; depthwise writing its
    intermediate, then pointwise), per workload, timed with HIP events on the stream."""
    import torch
    res = {}
    for w in wls:
        inp = w.inputs()
        t = {k: (None if v is None else torch.from_numpy(v).cuda()) for k, v in inp.items()}
        del inp
        p, d = w.params, w.dims
        fused_out = torch.empty(out_shape(w), device="cuda")
        if w.op == "conv3d_mish_tanh":
            inter = torch.empty(out_shape(w), device="cuda")

            def unfused():
                cf.conv3d_bias(t["x"], t["w"], t["b"], p["stride"], p["pad"], out=inter)
                cf.mish_tanh(inter, out=inter)
        elif w.op == "conv3d_div_maxpool_gap_bias_sum":
            od, oh, ow = out_dims(w)
            inter = torch.empty((d["N"], d["O"], od, oh, ow), device="cuda")

            def unfused():
                cf.conv3d_bias(t["x"], t["w"], t["conv_b"], out=inter)
                cf.div_maxpool_gap_bias_sum(inter, p["divisor"], p["pool"], t["bias"],
                                            out=fused_out)
        elif w.op == "dwsep_conv2d":
            ho, wo = out_dims(w)
            inter = torch.empty((d["N"], d["C"], ho, wo), device="cuda")
            if (p["stride"], p["dilation"]) != (1, 1):
                continue

            def unfused():
                cf.depthwise_conv2d(t["x"], t["dw_w"], t["dw_b"], p["stride"], p["pad"],
                                    p["dilation"], out=inter)
                cf.pointwise_conv2d(inter, t["pw_w"], t["pw_b"], out=fused_out)
        else:
            continue

        def timed(fn):
            for _ in range(warmup):
                fn()
            torch.cuda.synchronize()
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                  for _ in range(steps)]
            for a, b in ev:
                a.record()
                fn()
                b.record()
            torch.cuda.synchronize()
            return float(np.mean([a.elapsed_time(b) for a, b in ev]))

        ms_f = timed(lambda: run_op(cf, w, t, fused_out))
        ms_u = timed(unfused)
        macs, nbytes = work(w)
        res[w.name] = {"fused_ms": round(ms_f, 4), "unfused_ms": round(ms_u, 4),
                       "speedup": round(ms_u / ms_f, 3),
                       "intermediate_mb": round(inter.numel() * 4 / 1e6, 1),
                       "fused_tflops": round(2 * macs / ms_f / 1e9, 2)}
        del t, fused_out, inter
        torch.cuda.empty_cache()
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--reps", type=int, default=20,
                    help="launches per workload for the cold and the warm figures")
    ap.add_argument("--tiny-reps", type=int, default=200,
                    help="launches of the tiny configuration (0: skip it)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-frac", type=float, default=1.0,
                    help="fraction of each workload's batch the oracle baseline runs on")
    ap.add_argument("--workloads", default=",".join(map(str, BENCH_WORKLOADS)))
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="before the benchmark, run a device multiply over this many MiB "
                         "(3 times), so that rocprofv3 --pmc FETCH_SIZE/WRITE_SIZE of the same "
                         "run can be scaled to known bytes")
    ap.add_argument("--summarize-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="turn two rocprofv3 --pmc counter_collection.csv files (FETCH_SIZE, "
                         "WRITE_SIZE) of runs that included --copy-calibration-mib into "
                         "profiles/traffic.json")
    ap.add_argument("--calibration-mib", type=int, default=1024)
    ap.add_argument("--ceilings", action="store_true",
                    help="instead of the benchmark, measure the practical ceilings: an fp32 "
                         "MFMA issue loop with no memory traffic, and torch copy / fill over "
                         "1 GiB")
    ap.add_argument("--ablation", action="store_true",
                    help="instead of the benchmark, time each workload fused and unfused "
                         "(separate conv/epilogue/reduce or depthwise/pointwise kernels)")
    args = ap.parse_args()
    if args.summarize_traffic:
        summarize_traffic(*args.summarize_traffic, args.calibration_mib)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path "
              "(each batch item is independent, so batch sharding needs no communication). "
              "Run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import implicit_gemm_convolution_conv3d_amd as cf
    from implicit_gemm_convolution_conv3d_amd import workloads as wl

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration_mib:
        n = args.copy_calibration_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.mul(src, 2.0, out=dst)  # one elementwise kernel: reads n floats, writes n
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": 4 * n}), flush=True)
        del src, dst
        torch.cuda.empty_cache()
    cf.lib()  # fail loudly now if the library is missing
    dev = torch.device("cuda:0")
    ids = [int(s) for s in args.workloads.split(",") if s]
    wls = [wl.WORKLOADS[i] for i in ids]
    if args.ceilings:
        print(json.dumps({"ceilings": ceilings(cf, args.steps)}), flush=True)
        return
    if args.ablation:
        print(json.dumps({"ablation": ablation(cf, wls, args.steps, args.warmup),
                          "kernel_source_sha": kernel_source_sha()}), flush=True)
        return

    tensors, outs = [], []
    for w in wls:
        inp = w.inputs()
        tensors.append({k: (None if v is None else torch.from_numpy(v).to(dev))
                        for k, v in inp.items()})
        outs.append(torch.empty(out_shape(w), dtype=torch.float32, device=dev))
        del inp
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream(dev)
    for _ in range(args.warmup):
        for w, t, o in zip(wls, tensors, outs):
            run_op(cf, w, t, o)
    torch.cuda.synchronize()

    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in wls] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        for i, (w, t, o) in enumerate(zip(wls, tensors, outs)):
            ev[s][i][0].record(stream)
            run_op(cf, w, t, o)
            ev[s][i][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps

    step_ms = {w.name: np.array([ev[s][i][0].elapsed_time(ev[s][i][1])
                                 for s in range(args.steps)]) for i, w in enumerate(wls)}
    step_macs = sum(work(w)[0] for w in wls)
    value = 2 * step_macs / (ms_per_step * 1e-3) / 1e12

    # Per-workload figures, after the timed steps: each workload alone, `reps` launches with
    # the cache flushed before each (cold, the headline) and `reps` back-to-back (warm).
    flush = Flusher(torch, dev)
    per = {}
    for w, t, o in zip(wls, tensors, outs):
        cold = launch_times(torch, stream, lambda: run_op(cf, w, t, o), args.reps, flush)
        warm = launch_times(torch, stream, lambda: run_op(cf, w, t, o), args.reps, None)
        per[w.name] = workload_figures(w, cold, warm, step_ms[w.name], cf.last_kernel())
    if args.tiny_reps and 1 not in ids:
        # the tiny configuration: launch-bound, reported but not graded on throughput
        w1 = wl.WORKLOADS[1]
        t1 = {k: (None if v is None else torch.from_numpy(v).to(dev))
              for k, v in w1.inputs().items()}
        o1 = torch.empty(out_shape(w1), dtype=torch.float32, device=dev)
        for _ in range(args.warmup):
            run_op(cf, w1, t1, o1)
        cold = launch_times(torch, stream, lambda: run_op(cf, w1, t1, o1), args.tiny_reps, flush)
        warm = launch_times(torch, stream, lambda: run_op(cf, w1, t1, o1), args.tiny_reps, None)
        per[w1.name] = workload_figures(w1, cold, warm, None, cf.last_kernel())
        del t1, o1
    del flush

    # the roofline object: the kernel with the longest time in the timed steps, its
    # algorithmic FLOP per launch over its average launch time there
    dominant = max(wls, key=lambda w: float(step_ms[w.name].mean()))
    dom_ms = float(step_ms[dominant.name].mean())
    dmacs, _ = work(dominant)
    achieved = 2 * dmacs / (dom_ms * 1e-3) / 1e12
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_FP32_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_FP32_TFLOPS, 4),
                "traffic": load_traffic(dominant.name), "kernel": per[dominant.name]["kernel"],
                "workload": dominant.name}

    cpu = None
    if not args.no_cpu_baseline:
        del tensors, outs
        torch.cuda.empty_cache()
        base = list(wls)
        if args.tiny_reps and 1 not in ids:
            base = [wl.WORKLOADS[1]] + base
        v, cores, desc, cpu_per = cpu_baseline(base, args.cpu_sample_frac)
        cpu = {"value": round(v, 5), "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
               "sample": desc, "per_workload": cpu_per, **host_info()}

    line = {
        "metric": "conv TFLOP/s (2xMACs) and % fp32 MFMA/HBM roofline per config, 1xMI355X",
        "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": "fused conv hot path: " + " + ".join(w.name for w in wls),
                   "per_workload": per, "kernel_source_sha": kernel_source_sha()},
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


FLUSH_BYTES = 512 << 20   # twice the 256 MB last-level (MALL) cache


class Flusher:
    """Empties the caches between timed launches: writes one 512 MiB buffer, then reads
    another 512 MiB, so the caches end up holding clean lines of an unrelated buffer (a write
    alone would leave dirty lines that the timed kernel would have to write back)."""

    def __init__(self, torch, dev):
        self.w = torch.empty(FLUSH_BYTES // 4, dtype=torch.float32, device=dev)
        self.r = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device=dev)
        self.s = torch.empty((), dtype=torch.float32, device=dev)
        self.torch = torch

    def __call__(self, rep):
        self.w.fill_(float(rep))
        self.torch.sum(self.r, dim=0, out=self.s)


def launch_times(torch, stream, fn, reps, flush):
    """Milliseconds of `reps` launches of fn, each between two HIP events on the launch
    stream; flush (if given) runs before each launch, outside its events.  The same number of
    launches (flushed alike) runs first, untimed: the first few dozen launches of a workload
    after another one ran measure up to 15 % slower than the steady state."""
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(reps)]
    for r in range(reps):
        if flush is not None:
            flush(r)
        fn()
    for r, (a, b) in enumerate(ev):
        if flush is not None:
            flush(r)
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    return np.array([a.elapsed_time(b) for a, b in ev])


def workload_figures(w, cold, warm, step, launched=None):
    """Per-workload record: the cold median is the headline time; rates and roofline
    fractions are computed from it.  `launched`: the kernel the library reported launching
    (convfuse_last_kernel), else the dispatch rules' expectation."""
    macs, nbytes = work(w)
    gmacs = gemm_macs(w)
    med = float(np.median(cold))
    sec = med * 1e-3
    fm = 2 * gmacs / sec / 1e12 / PEAK_FP32_TFLOPS
    fh = nbytes / sec / 1e9 / PEAK_HBM_GBS
    rec = {
        "op": w.op, "kernel": launched or kernel_name(w), "reps": int(cold.size),
        "ms_median": round(med, 4), "ms_min": round(float(cold.min()), 4),
        "ms_mean": round(float(cold.mean()), 4),
        "ms_warm_median": round(float(np.median(warm)), 4),
        "ms_in_step_mean": None if step is None else round(float(step.mean()), 4),
        "tflops": round(2 * macs / sec / 1e12, 2),
        "gflop": round(2 * macs / 1e9, 3),
        "mfma_gflop": round(2 * gmacs / 1e9, 3),
        "vector_gflop": round(2 * (macs - gmacs) / 1e9, 3),
        "frac_fp32_mfma": round(fm, 4),
        "gbs": round(nbytes / sec / 1e9, 1), "mbytes": round(nbytes / 1e6, 2),
        "frac_hbm": round(fh, 4),
        # max(matrix FLOP / matrix peak, bytes / HBM peak) / time
        "frac_roofline": round(max(fm, fh), 4),
    }
    if w.index == 1:
        rec["graded"] = None  # launch-bound: parity only
    else:
        bound = graded_bound(w)
        frac, target = (fh, 0.60) if bound == "hbm" else (fm, 0.50)
        rec["graded"] = {"bound": bound, "frac": round(frac, 4), "target": target,
                         "met": bool(frac >= target)}
    return rec


if __name__ == "__main__":
    main()
