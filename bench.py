"""Benchmark: orthogonalized params/s and MFMA TFLOP/s on the Llama-3-8B layer set.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload llama3_8b]

A step is one megabatched orthogonalization call over all 224 momentum matrices
of the 32-layer Llama-3-8B layer set (q,o 4096x4096; k,v 1024x4096; gate,up
14336x4096; down 4096x14336), bf16, rank-64 + 0.05 noise with per-matrix scale
10^U(-3,0), 5 Gram Newton-Schulz iterations with restarts every 2.  Inputs are
synthetic and resident in HBM before the timed region.  Prints one JSON line.

Beside the GPU figures: a roofline entry for the dominant kernel (the one with
the most GPU time: algorithmic FLOPs per launch over its average launch time,
measured with hipEvents on the launch stream by the library's profiling hook,
against the dense fp16/bf16 MFMA peak; for a streaming pass, algorithmic bytes
against HBM), and the fp64 CPU oracle timed on a bounded sample of the same
workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_MFMA16_TFLOPS = 2516.6   # MI355X dense fp16 / bf16 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
PEAK_MFMA32_TFLOPS = 157.3    # MI355X dense fp32 matrix
PEAK_FP64_TFLOPS = 78.6       # MI355X fp64 vector FMA (the FP64 path's k_gemm64)
LOWRANK_RANK, LOWRANK_BETA = 256, 0.1


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="llama3_8b", choices=["llama3_8b", "gpt2_small", "llama3_70b",
                                                                "llama3_8b_rows", "llama3_8b_lowrank",
                                                                "fp32_64x128"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--update", action="store_true",
                    help="row-subset workload only: fuse the weight update into the step (bf16 weights, "
                         "lr 0.02 times sqrt(max(1, rows/cols)), weight decay 0.1)")
    ap.add_argument("--cpu-sample-seconds", type=float, default=20.0)
    ap.add_argument("--workspace-gib", type=float, default=None,
                    help="cap the workspace at this many GiB: the batch runs in waves of matrices that fit it")
    ap.add_argument("--summarize", metavar="DIR",
                    help="print a text summary of the rocprofv3 CSV output under DIR and exit")
    ap.add_argument("--copy-ceiling", action="store_true",
                    help="time passes that read and write 1, 4 and 16 GiB once (runtime copy, elementwise kernel; the rate a streaming pass "
                         "that reads and writes each byte once can reach) and exit")
    ap.add_argument("--gemm-ceiling", action="store_true",
                    help="time the vendor library's dense GEMMs (torch.matmul: hipBLASLt/rocBLAS) in fp16 and "
                         "bf16 on random and on constant operands at the Llama-3-8B product shapes, each "
                         "sustained for about two seconds (the power limit's steady state), and exit")
    ap.add_argument("--profile", action="store_true",
                    help="only run warmup + steps (for rocprofv3), no baseline; also runs one plain 1 GiB "
                         "device copy so byte counters can be calibrated against a known size")
    return ap.parse_args()


def make_inputs(wl, torch):
    import workloads as W
    if wl.name in ("llama3_8b", "llama3_8b_rows"):
        return W.llama3_8b_torch(step=1 if wl.name.endswith("rows") else None)
    if wl.name == "gpt2_small":
        import numpy as np
        return [torch.from_numpy(W.bf16_bits_to_f32(b)).cuda().to(torch.bfloat16) for b in W.gpt2_small_np()]
    if wl.name == "llama3_70b":
        return W.llama3_70b_torch()
    if wl.name == "fp32_64x128":
        return [torch.from_numpy(W.fp32_64x128()).cuda()]
    raise ValueError(wl.name)


def cpu_baseline(wl, Ms, seconds, torch):
    """Oracle (fp64 numpy) on a bounded sample: whole matrices of the workload
    in batch order until about `seconds` of CPU work; params/s = sampled
    params / wall time."""
    import numpy as np
    from oracle import dion_oracle as O
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [os.cpu_count()])
    except Exception:
        cores = os.cpu_count()
    kw = wl.ns_kwargs()
    step_mode = wl.name.endswith("rows")
    # sample: layer 0's k and v (1024x4096), then q (4096x4096), then o, ... until the budget
    order = [1, 2, 0, 3, 4, 5, 6] if len(Ms) >= 7 else list(range(len(Ms)))
    done, params, t_total = [], 0, 0.0
    for i in order:
        M = Ms[i].float().cpu().numpy()
        t0 = time.perf_counter()
        if step_mode:   # the whole step from a zero buffer: momentum, selection, Gram-NS, write-out
            O.rowsubset_step([np.zeros(M.shape, np.float32)], [M], wl.beta, **kw)
        else:
            O.orthogonalize(M, **kw)
        t_total += time.perf_counter() - t0
        params += M.shape[0] * M.shape[1]
        done.append(f"{M.shape[0]}x{M.shape[1]}")
        if t_total >= seconds:
            break
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), model)
    except OSError:
        pass
    nproc = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    return {"value": params / t_total, "unit": "params/s", "cores": int(cores), "nproc": int(nproc),
            "cpu_model": model, "kind": "oracle",
            "sample": f"{len(done)} whole matrices of layer 0 ({', '.join(done)}; {params/1e6:.1f}M params), "
                      + ("one full row-subset step each (fp32 momentum, selection, fp64 Gram-NS of the selected "
                         "rows)" if step_mode else "full fp64 Gram-NS") +
                      f" with the workload's hyper-parameters, {t_total:.1f} s"}


# the kernels and the plan that decides what each launch of them covers
KERNEL_SOURCES = ("orthogonalized_optimizer_step_amd/csrc/gemm_kernels.hip",
                  "orthogonalized_optimizer_step_amd/csrc/stream_kernels.hip",
                  "orthogonalized_optimizer_step_amd/csrc/tiny_kernels.hip",
                  "orthogonalized_optimizer_step_amd/csrc/lowrank_gemm.hip",
                  "orthogonalized_optimizer_step_amd/csrc/lowrank_kernels.hip",
                  "orthogonalized_optimizer_step_amd/csrc/lowrank_internal.h",
                  "orthogonalized_optimizer_step_amd/csrc/dion_api.cpp",
                  "orthogonalized_optimizer_step_amd/csrc/dion_internal.h")
# counter summaries per workload (the TRAFFIC lines of a file hold only for the workload it was taken on)
TRAFFIC_FILES = {"llama3_8b": os.path.join(ROOT, "profiles", "llama3_8b_hbm_traffic.txt"),
                 "llama3_8b_rows": os.path.join(ROOT, "profiles", "llama3_8b_rows_hbm_traffic.txt"),
                 "llama3_8b_rows+update": os.path.join(ROOT, "profiles", "llama3_8b_rows_update_hbm_traffic.txt"),
                 "llama3_8b_lowrank": os.path.join(ROOT, "profiles", "llama3_8b_lowrank_hbm_traffic.txt")}


def sources_sha256():
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    return h.hexdigest()


def short_kernel(name):
    """Kernel name without its parameter list (template arguments kept)."""
    depth, out = 0, []
    for ch in name:
        if ch == "(" and depth == 0:
            break
        depth += ch == "<"
        depth -= ch == ">"
        out.append(ch)
    return "".join(out).replace("void ", "").strip('"')


def summarize(d):
    """Text summary of rocprofv3 --output-format csv results under d: the
    kernel statistics, or per-kernel averages of collected counters.  HBM
    byte counters (FETCH_SIZE, WRITE_SIZE, KiB per dispatch) are scaled by
    what the same counter reads for the plain 1 GiB calibration copy that
    bench.py --profile runs, and emitted as TRAFFIC lines for bench.py."""
    import collections
    import csv
    import glob
    stats = glob.glob(os.path.join(d, "**", "*kernel_stats.csv"), recursive=True)
    ctrs = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    traces = glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True)
    if stats:
        # per-dispatch durations in launch order, for the average after the first
        # dispatch (the warmup call's, when the kernel runs once per call)
        per = collections.defaultdict(list)
        for f in traces:
            for r in sorted(csv.DictReader(open(f)), key=lambda r: int(r["Start_Timestamp"])):
                per[short_kernel(r["Kernel_Name"])].append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
        rows = list(csv.DictReader(open(stats[0])))
        print(f"{'kernel':64s} {'calls':>6s} {'total ms':>10s} {'avg us':>11s} {'%':>6s} {'avg us after 1st':>17s}")
        for r in rows:
            k = short_kernel(r["Name"])
            ds = per.get(k, [])
            rest = f"{sum(ds[1:]) / len(ds[1:]) / 1e3:17.1f}" if len(ds) > 1 else f"{'-':>17s}"
            print(f"{k[:64]:64s} {int(r['Calls']):6d} {float(r['TotalDurationNs'])/1e6:10.3f} "
                  f"{float(r['AverageNs'])/1e3:11.1f} {float(r['Percentage']):6.2f} {rest}")
    for f in ctrs:
        rows = list(csv.DictReader(open(f)))
        agg = collections.defaultdict(lambda: collections.defaultdict(list))
        for r in rows:
            agg[short_kernel(r["Kernel_Name"])][r["Counter_Name"]].append(float(r["Counter_Value"]))
        calib = {}
        for k, cs in agg.items():
            if "copyBuffer" in k:
                for c, v in cs.items():
                    # the 1 GiB copy (counters in KiB; FETCH_SIZE reads about half of it),
                    # far above the per-call uploads of a few KiB
                    big = [x for x in v if x > (1 << 18)]
                    if big:
                        calib[c] = (1 << 20) / max(big)      # true KiB / counted KiB
        print(f"\n{'kernel':64s} {'counter':12s} {'dispatches':>10s} {'avg GiB/dispatch':>17s} {'scaled':>8s}")
        for k, cs in sorted(agg.items()):
            for c, v in sorted(cs.items()):
                avg = sum(v) / len(v) / (1 << 20)
                sc = calib.get(c, 1.0)
                print(f"{k[:64]:64s} {c:12s} {len(v):10d} {avg:17.3f} {avg * sc:8.3f}")
                if c in ("FETCH_SIZE", "WRITE_SIZE") and "dion::" in k:
                    print("TRAFFIC " + json.dumps({"kernel": k, "counter": c, "bytes_per_dispatch": avg * sc * (1 << 30),
                                                   "scale": sc, "sources_sha256": sources_sha256()}))
        if calib:
            print("\ncalibration (true / counted, from the 1 GiB copy): " +
                  ", ".join(f"{c} x{v:.3f}" for c, v in calib.items()))
        clock_table(rows, traces)


def clock_table(rows, traces):
    """Per-kernel range of the GPU clock and MFMA busy fraction over the
    dispatches of a counter run that holds GRBM_GUI_ACTIVE (summed over the 8
    XCDs) and SQ_VALU_MFMA_BUSY_CYCLES (summed over the 1024 SIMDs).  The
    dispatch duration comes from the counter rows' own timestamps, else from
    a kernel trace of the same run, joined by dispatch id."""
    import collections
    import csv
    if not any(r["Counter_Name"] == "GRBM_GUI_ACTIVE" for r in rows):
        return
    disp = collections.defaultdict(dict)
    for r in rows:
        e = disp[(r["Kernel_Name"], r["Dispatch_Id"])]
        e[r["Counter_Name"]] = e.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
        if r.get("Start_Timestamp") and r.get("End_Timestamp"):
            e["ns"] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
    ns = {}
    for f in traces:
        for r in csv.DictReader(open(f)):
            ns[r["Dispatch_Id"]] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
    per = collections.defaultdict(list)
    for (name, did), e in disp.items():
        dur = e.get("ns") or ns.get(did)
        if not dur or "GRBM_GUI_ACTIVE" not in e:
            continue
        cyc = e["GRBM_GUI_ACTIVE"] / 8.0
        busy = e.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / cyc / 1024.0 if cyc else 0.0
        per[short_kernel(name)].append((cyc / dur, busy))
    if not per:
        print("\n(no dispatch durations: run the counters with --kernel-trace for the clock table)")
        return
    print(f"\n{'kernel':42s} {'disp':>5s} {'clock GHz':>12s} {'MFMA busy':>11s} {'clock x busy':>12s}")
    for k, v in sorted(per.items(), key=lambda kv: sum(b for _, b in kv[1]) / len(kv[1])):
        ghz = [g for g, _ in v]
        busy = [b for _, b in v]
        prod = sum(g * b for g, b in v) / len(v)
        print(f"{k[:42]:42s} {len(v):5d} {min(ghz):5.2f}-{max(ghz):5.2f}  {min(busy):4.2f}-{max(busy):5.2f} {prod:12.2f}")


def traffic_for(kernel, workload):
    """HBM bytes per launch (fetch + write) of `kernel` from the committed
    counter summary of `workload`, or None if absent or taken on different
    kernel sources."""
    path = TRAFFIC_FILES.get(workload)
    if path is None or not os.path.exists(path):
        return None
    sha = sources_sha256()
    got = {}
    for line in open(path):
        if line.startswith("TRAFFIC {"):
            t = json.loads(line[8:])
            if t["kernel"] == kernel and t["sources_sha256"] == sha:
                got[t["counter"]] = t["bytes_per_dispatch"]
    if "FETCH_SIZE" in got and "WRITE_SIZE" in got:
        return got["FETCH_SIZE"] + got["WRITE_SIZE"]
    return None


def cpu_baseline_lowrank(grads, Qs, seconds):
    """The low-rank oracle on whole matrices of layer 0 (k, v, q, ...) until
    about `seconds` of CPU work; params/s = sampled params / wall time."""
    import numpy as np
    from oracle import orthdion_oracle as L
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [os.cpu_count()])
    except Exception:
        cores = os.cpu_count()
    done, params, t_total = [], 0, 0.0
    for i in [1, 2, 0, 3, 4, 5, 6]:
        G = grads[i].float().cpu().numpy()
        M = np.zeros_like(G)
        Q = Qs[i].cpu().numpy()
        t0 = time.perf_counter()
        L.lowrank_step(M, G, Q, LOWRANK_BETA, "qr")
        t_total += time.perf_counter() - t0
        params += G.shape[0] * G.shape[1]
        done.append(f"{G.shape[0]}x{G.shape[1]}")
        if t_total >= seconds:
            break
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), model)
    except OSError:
        pass
    nproc = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    return {"value": params / t_total, "unit": "params/s", "cores": int(cores), "nproc": int(nproc),
            "cpu_model": model, "kind": "oracle",
            "sample": f"{len(done)} whole matrices of layer 0 ({', '.join(done)}; {params/1e6:.1f}M params), "
                      f"one fp64 Orth-Dion step at rank {LOWRANK_RANK}, {t_total:.1f} s"}


def time_plain(torch, call, steps):
    """ms per step of `steps` more calls with the library's profiling events
    off: the timed region above records two hipEvents around every launch,
    which costs a few microseconds each (about 12% of the 1.6 ms GPT-2 batch,
    0.1% of the Llama-3-8B call)."""
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for _ in range(steps):
        call()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps


def calibration_copy(torch, dev):
    """The runtime's copy of exactly 1 GiB (read and written once), whose byte
    counters scale the counters of the library's kernels in a --profile run."""
    src = torch.empty(1 << 28, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def bench_lowrank(args, torch, dion):
    """One Orth-Dion step (rank 256, beta 0.1) over the Llama-3-8B layer set:
    bf16 gradients of one step, fp32 buffers from zero, seeded Gaussian right
    factors, bf16 updates."""
    import workloads as W
    dev = torch.device("cuda:0")
    grads = W.llama3_8b_torch(step=1)
    shapes = [tuple(g.shape) for g in grads]
    Ms = [torch.zeros(s, dtype=torch.float32, device=dev) for s in shapes]
    gen = torch.Generator(device=dev)
    gen.manual_seed(21)
    Qs = [torch.randn(c, min(LOWRANK_RANK, r, c), generator=gen, device=dev) for r, c in shapes]
    Q0 = [Q.clone() for Q in Qs] if not args.no_cpu_baseline else None
    outs = [torch.empty(s, dtype=torch.bfloat16, device=dev) for s in shapes]
    ws = torch.empty(dion.lowrank_workspace_size(shapes, LOWRANK_RANK) + 256, dtype=torch.uint8, device=dev)
    call = lambda: dion.lowrank_step(Ms, grads, Qs, LOWRANK_BETA, mode="qr", outs=outs, workspace=ws)  # noqa: E731
    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    if args.profile:
        calibration_copy(torch, dev)
    dion.profile_enable(True)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record()
    for _ in range(args.steps):
        call()
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_total = start.elapsed_time(end)
    recs = dion.profile_records()
    dion.profile_enable(False)
    ms_per_step = ms_total / args.steps
    if args.profile:
        print(json.dumps({"ms_per_step": ms_per_step}))
        return
    ms_plain = time_plain(torch, call, args.steps)
    phases, kernels = {}, {}
    for name, kern, ms, u, r, b, a in recs:
        for key, tab in ((name, phases), (kern, kernels)):
            e = tab.setdefault(key, {"ms": 0.0, "launches": 0, "useful": 0.0, "bytes": 0.0})
            e["ms"] += ms
            e["launches"] += 1
            e["useful"] += u
            e["bytes"] += b
    dom = max((k for k, v in kernels.items() if v["useful"] > 0), key=lambda k: kernels[k]["ms"])
    d = kernels[dom]
    avg_ms = d["ms"] / d["launches"]
    useful_rate = (d["useful"] / d["launches"]) / (avg_ms * 1e-3) / 1e12
    # the products are fp32 GEMMs computed on 16-bit matrix cores: two fp16
    # terms per operand (three MFMA products) or, for the instances whose
    # template flag is false, three bf16 terms (six); the bf16 update reads
    # one fp16 term (one product): priced as the MFMA work they execute
    terms = 6 if dom.endswith("false>") else (1 if dom.endswith("dma<1>") else 3)
    achieved = useful_rate * terms
    useful = sum(v["useful"] for v in phases.values()) / args.steps
    params = sum(r * c for r, c in shapes)
    line = {
        "metric": f"low-rank Orth-Dion updated params/sec (rank {LOWRANK_RANK}), Llama-8B layer set",
        "value": params * args.steps / (ms_total * 1e-3),
        "unit": "params/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"llama3_8b_lowrank: {len(shapes)} matrices, {params/1e9:.3f} G params, "
                               f"Orth-Dion (QR), rank {LOWRANK_RANK}, beta {LOWRANK_BETA}, bf16 gradients and update",
                   "matrices": len(shapes), "params": params, "rank": LOWRANK_RANK},
        "useful_tflops": useful / (ms_per_step * 1e-3) / 1e12,
        "host_wall_s": wall,
        "ms_per_step_uninstrumented": ms_plain,
        "roofline": {"bound": "mfma", "kernel": dom, "achieved": achieved, "peak": PEAK_MFMA16_TFLOPS,
                     "unit": "TFLOP/s", "frac": achieved / PEAK_MFMA16_TFLOPS,
                     "traffic": traffic_for(dom, "llama3_8b_lowrank"),
                     "launch_ms": avg_ms, "useful_flops_per_launch": d["useful"] / d["launches"],
                     "mfma_products_per_useful": terms,
                     "useful_fp32_tflops": useful_rate, "fp32_matrix_peak": PEAK_MFMA32_TFLOPS,
                     "algorithmic_bytes_per_launch": d["bytes"] / d["launches"]},
        "phases": {n: {"ms_per_step": round(p["ms"] / args.steps, 3),
                       "launches_per_step": p["launches"] // args.steps,
                       **({"tflops": round(p["useful"] / (p["ms"] * 1e-3) / 1e12, 1)} if p["useful"] else
                          {"gbs": round(p["bytes"] / (p["ms"] * 1e-3) / 1e9, 1)})}
                   for n, p in sorted(phases.items(), key=lambda kv: -kv[1]["ms"])},
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline_lowrank(grads, Q0, args.cpu_sample_seconds)
    print(json.dumps(line))


def copy_ceiling(torch, reps=10):
    """HBM rate of a pass that reads and writes each byte once, counting both:
    the runtime's device copy (torch copy_, a hipMemcpy kernel) and PyTorch's
    vectorized elementwise kernel (dst = src * 1).  One JSON line per kind
    and size, the median of `reps` timed passes."""
    for kind in ("copy", "elementwise"):
        for gib in (1, 4, 16):
            n = (gib << 30) // 4
            src = torch.empty(n, dtype=torch.float32, device="cuda").fill_(1.0)
            dst = torch.empty_like(src)
            op = (lambda: dst.copy_(src)) if kind == "copy" else (lambda: torch.mul(src, 1.0, out=dst))
            for _ in range(2):
                op()
            times = []
            for _ in range(reps):
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record()
                op()
                b.record()
                b.synchronize()
                times.append(a.elapsed_time(b))
            times.sort()
            ms = times[len(times) // 2]
            print(json.dumps({"copy_ceiling": {"kind": kind, "gib": gib, "bytes_moved": 2 * (gib << 30), "ms": ms,
                                               "gbs": 2 * (gib << 30) / ms / 1e6, "min_ms": times[0]}}), flush=True)
            del src, dst
            torch.cuda.empty_cache()


def gemm_ceiling(torch, seconds=2.0):
    """Dense-GEMM throughput of the vendor library on the GPU it runs on, as a
    ceiling for the hand-written kernels measured on the same device: torch.matmul (hipBLASLt / rocBLAS,
    fp32 accumulate) in fp16 and bf16, on N(0,1) operands (full-entropy
    significands, like the iterates) and on constant operands (few toggling
    bits), at the products of the Llama-3-8B set: 4096^3 (an m x m chain
    product), 4096 x 4096 x 14336 (a Gram with a long reduction) and
    4096 x 14336 x 4096 (a tall apply).  Each shape runs back to back for about
    `seconds` so that the board reaches its power limit; the rate is the
    median over ten equal slices of that run, timed with hipEvents on the
    current stream.  One JSON line per dtype, data and shape."""
    shapes = [(4096, 4096, 4096), (4096, 14336, 4096), (4096, 4096, 14336)]
    for dt_name, dt in (("fp16", torch.float16), ("bf16", torch.bfloat16)):
        for data in ("random", "constant"):
            for (m, k, n) in shapes:
                g = torch.Generator(device="cuda").manual_seed(7)
                if data == "random":
                    a = torch.randn((m, k), generator=g, device="cuda").to(dt)
                    b = torch.randn((k, n), generator=g, device="cuda").to(dt)
                else:
                    a = torch.full((m, k), 0.5, device="cuda", dtype=dt)
                    b = torch.full((k, n), 0.25, device="cuda", dtype=dt)
                c = torch.empty((m, n), device="cuda", dtype=dt)
                flop = 2.0 * m * n * k
                for _ in range(3):
                    torch.matmul(a, b, out=c)
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                torch.matmul(a, b, out=c)
                e1.record()
                e1.synchronize()
                per = max(e0.elapsed_time(e1), 1e-3)
                reps = max(1, int(seconds * 1e3 / per / 10))
                times = []
                for _ in range(10):
                    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    e0.record()
                    for _ in range(reps):
                        torch.matmul(a, b, out=c)
                    e1.record()
                    e1.synchronize()
                    times.append(e0.elapsed_time(e1) / reps)
                first = times[0]
                times.sort()
                ms = times[len(times) // 2]
                print(json.dumps({"gemm_ceiling": {"dtype": dt_name, "data": data, "m": m, "k": k, "n": n,
                                                   "ms": ms, "tflops": flop / ms / 1e9,
                                                   "first_slice_tflops": flop / first / 1e9,
                                                   "frac_of_dense_peak": flop / ms / 1e9 / 2516.6,
                                                   "reps_per_slice": reps}}), flush=True)
                del a, b, c
                torch.cuda.empty_cache()


def main():
    args = parse()
    if args.summarize:
        summarize(args.summarize)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "one GPU only: --gpus must be 1 (across GPUs the path would shard by "
                                   "whole matrix, with no collective inside the orthogonalization)"}))
        sys.exit(2)
    import torch
    if args.copy_ceiling:
        copy_ceiling(torch)
        return
    if args.gemm_ceiling:
        gemm_ceiling(torch)
        return
    import orthogonalized_optimizer_step_amd as dion
    from workloads import WORKLOADS

    if args.workload == "llama3_8b_lowrank":
        torch.cuda.init()
        bench_lowrank(args, torch, dion)
        return
    wl = WORKLOADS[args.workload]
    torch.cuda.init()
    dev = torch.device("cuda:0")
    Ms = make_inputs(wl, torch)
    step_mode = wl.name.endswith("rows")
    budget = int(args.workspace_gib * (1 << 30)) if args.workspace_gib else None
    orth = dion.Orthogonalizer(wl.shapes, wl.dtype, wl.coeffs, wl.n_iter, wl.restart_every, wl.restart_mask,
                               wl.safety, wl.row_frac, "auto", device=dev, step_mode=step_mode,
                               workspace_budget=budget)
    if args.update and not step_mode:
        print(json.dumps({"error": "--update needs the row-subset workload (llama3_8b_rows)"}))
        sys.exit(2)
    if step_mode and args.update:
        Es = [torch.zeros(M.shape, dtype=torch.float32, device=dev) for M in Ms]
        g = torch.Generator(device=dev)
        g.manual_seed(11)
        Ws = [(torch.randn(M.shape, generator=g, device=dev) * 0.02).to(torch.bfloat16) for M in Ms]
        alphas = [0.02 * max(1.0, r / c) ** 0.5 for r, c in wl.shapes]
        call = lambda: orth.step_update(Es, Ms, Ws, wl.beta, alphas, 0.02 * 0.1)  # noqa: E731
    elif step_mode:
        Es = [torch.zeros(M.shape, dtype=torch.float32, device=dev) for M in Ms]
        outs = [torch.empty_like(M) for M in Ms]
        call = lambda: orth.step(Es, Ms, outs, wl.beta)  # noqa: E731
    else:
        outs = [torch.empty_like(M) for M in Ms]
        call = lambda: orth(Ms, outs)  # noqa: E731
    torch.cuda.synchronize()

    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    if args.profile:
        calibration_copy(torch, dev)

    dion.profile_enable(True)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record()
    for _ in range(args.steps):
        call()
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_total = start.elapsed_time(end)
    recs = dion.profile_records()
    dion.profile_enable(False)
    ms_per_step = ms_total / args.steps
    if args.profile:
        print(json.dumps({"ms_per_step": ms_per_step}))
        return
    ms_plain = time_plain(torch, call, args.steps)

    params = wl.params
    useful = orth.useful_flops()
    # per-phase aggregation
    phases = {}
    for name, kern, ms, u, r, b, a in recs:
        ph = phases.setdefault(name, {"ms": 0.0, "launches": 0, "useful": 0.0, "mfma": 0.0, "bytes": 0.0,
                                      "kernels": set()})
        ph["kernels"].add(kern)
        ph["ms"] += ms
        ph["launches"] += 1
        ph["useful"] += u
        ph["mfma"] += r
        ph["bytes"] += b
    # the roofline entry is for the kernel instance with the most GPU time:
    # an MFMA kernel against the matrix peak, a streaming pass against HBM
    kernels = {}
    for name, kern, ms, u, r, b, a in recs:
        k = kernels.setdefault(kern, {"ms": 0.0, "launches": 0, "useful": 0.0, "alg": 0.0, "mfma": 0.0,
                                      "bytes": 0.0, "phases": set()})
        k["phases"].add(name)
        k["ms"] += ms
        k["launches"] += 1
        k["useful"] += u
        k["alg"] += a
        k["mfma"] += r
        k["bytes"] += b
    dom_kernel = max(kernels, key=lambda k: kernels[k]["ms"])
    d = kernels[dom_kernel]
    avg_ms = d["ms"] / d["launches"]
    compute = d["mfma"] > 0
    # an MFMA kernel is priced by its algorithmic FLOPs: the per-unit formulas
    # of the useful count over every product its launches run (the useful count
    # leaves out the accumulated restart factor and the restarts a cut
    # schedule adds, which this kernel instance also runs)
    achieved = ((d["alg"] / d["launches"]) / (avg_ms * 1e-3) / 1e12 if compute else
                (d["bytes"] / d["launches"]) / (avg_ms * 1e-3) / 1e9)
    # algorithmic HBM bytes per launch, from the plan: each operand term read
    # once and the result written once
    alg_bytes = d["bytes"] / d["launches"]
    traffic = traffic_for(dom_kernel, wl.name + ("+update" if args.update else ""))
    raw_total = sum(p["mfma"] for p in phases.values()) / args.steps
    phase_summary = {n: {"ms_per_step": round(p["ms"] / args.steps, 3),
                         "launches_per_step": p["launches"] // args.steps,
                         **({"useful_tflops": round(p["useful"] / (p["ms"] * 1e-3) / 1e12, 1),
                             "mfma_tflops": round(p["mfma"] / (p["ms"] * 1e-3) / 1e12, 1)} if p["mfma"] else
                            {"gbs": round(p["bytes"] / (p["ms"] * 1e-3) / 1e9, 1)})}
                     for n, p in sorted(phases.items(), key=lambda kv: -kv[1]["ms"])}
    value = params * args.steps / (ms_total * 1e-3)
    fp64 = wl.dtype == "fp32"   # fp32 momentum runs the FP64 path: fp64 FMA tiles, no MFMA
    peak = PEAK_FP64_TFLOPS if fp64 else PEAK_MFMA16_TFLOPS
    line = {
        "metric": "orthogonalized params/sec and MFMA TFLOP/s (% peak), Llama-8B layer set",
        "value": value,
        "unit": "params/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f64" if fp64 else "f16",
        "data": "synthetic",
        "config": {"workload": f"{wl.name}{' + fused weight update' if args.update else ''}: "
                               f"{len(wl.shapes)} matrices, {params/1e9:.3f} G params, "
                               f"K={wl.n_iter}, restart_every={wl.restart_every}, restart_mask={wl.restart_mask}, "
                               f"safety={wl.safety}, row_frac={wl.row_frac}",
                   "matrices": len(wl.shapes), "params": params, "n_iter": wl.n_iter,
                   **({"workspace_bytes": orth.ws_bytes} if budget else {})},
        "useful_tflops": useful / (ms_per_step * 1e-3) / 1e12,
        "useful_pct_peak": 100.0 * useful / (ms_per_step * 1e-3) / 1e12 / peak,
        "mfma_tflops": raw_total / (ms_per_step * 1e-3) / 1e12,
        "host_wall_s": wall,
        "ms_per_step_uninstrumented": ms_plain,
        "roofline": ({"bound": "alu" if fp64 else "mfma", "kernel": dom_kernel,
                      "phase": "+".join(sorted(d["phases"])), "achieved": achieved,
                      "peak": peak, "unit": "TFLOP/s", "frac": achieved / peak,
                      "traffic": traffic, "launch_ms": avg_ms,
                      "algorithmic_flops_per_launch": d["alg"] / d["launches"],
                      "useful_flops_per_launch": d["useful"] / d["launches"],
                      "useful_tflops": d["useful"] / d["launches"] / (avg_ms * 1e-3) / 1e12,
                      "mfma_tflops": d["mfma"] / d["launches"] / (avg_ms * 1e-3) / 1e12,
                      "algorithmic_bytes_per_launch": alg_bytes} if compute else
                     {"bound": "hbm", "kernel": dom_kernel, "phase": "+".join(sorted(d["phases"])),
                      "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": achieved / PEAK_HBM_GBS,
                      "traffic": traffic, "launch_ms": avg_ms, "algorithmic_bytes_per_launch": alg_bytes}),
        "phases": phase_summary,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(wl, Ms, args.cpu_sample_seconds, torch)
    print(json.dumps(line))


if __name__ == "__main__":
    main()
