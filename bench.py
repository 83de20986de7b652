"""Throughput of the fused cascaded GEMM on one MI355X.

A step is one fused cascade D = rnd(rnd(A.B0).B1)[.B2] over one batch of the
workload (one kernel launch).  Inputs are seeded synthetic tensors already in
HBM; the timed loop rotates over enough copies of them (>= 1 GiB in total, four
times the 256 MB Infinity Cache) that every step reads A and writes D in HBM.

With no --config the run measures the metric per dtype at the largest
workload of each: the headline is the three-GEMM fp16 cascade (workload 5),
and `per_dtype` adds the bf16 (workload 3) and fp64 (workload 4) ones.  Each
is timed as `repeats` blocks of --steps back-to-back launches (events on the
launch stream around each block; at least five blocks and 50 ms in all); the
median block gives ms_per_step, min and max are reported beside it.

Prints one JSON line: TFLOP/s of the whole job, the dominant kernel's
roofline figures (algorithmic bytes or FLOP over its measured duration), the
fractions of the measured matrix-core and HBM ceilings (kernels of the same
library that run only matrix instructions, only a copy stream, or a stream of
the workload's own A and D bytes over its own buffers), and the CPU oracle
timed on a bounded sample of the same workload.

--summarize-trace FILE reads a rocprofv3 kernel trace (CSV) and prints, per
kernel, the median, min and max duration of the last N launches (the timed
ones), for the profile summaries.
"""
import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

# dense MFMA, FLOP/s; tf32 has no matrix instruction on gfx950 and runs as
# bf16 passes, so its peak is the bf16 peak over the passes per product
PEAK = {"f16": 2516.6e12, "bf16": 2516.6e12, "f64": 78.6e12, "tf32": 2516.6e12 / 3, "tf32x4": 2516.6e12 / 4}
HBM = 8.0e12                                                   # B/s
ELT = {"f16": 2, "bf16": 2, "f64": 8, "tf32": 4, "fp8": 1}
# the largest workload of each dtype: the headline (fp16) and the others
HEADLINE = 5
PER_DTYPE = {"f16": 5, "bf16": 3, "f64": 4}


def workload_numbers(c, types=None):
    """FLOP and algorithmic bytes (A + weights + D) of a step; types: one per
    GEMM and D's, when the stages differ."""
    dims, b, M = c["dims"], c["batch"], c["M"]
    t = types or [c["dtype"]] * len(dims)
    flop = 2.0 * b * M * sum(dims[s] * dims[s + 1] for s in range(len(dims) - 1))
    wbytes = b * sum(dims[s] * dims[s + 1] * ELT[t[s]] for s in range(len(dims) - 1))
    byts = b * M * dims[0] * ELT[t[0]] + wbytes + b * M * dims[-1] * ELT[t[-1]]
    return flop, byts


def roofline(flop, algo_bytes, launch_ms, peak):
    """The binding roof of a kernel from its arithmetic intensity against the
    ridge point, and the fraction of it the measured launch reaches."""
    if flop / algo_bytes < peak / HBM:
        roof = {"bound": "hbm", "achieved": algo_bytes / (launch_ms * 1e-3) / 1e9, "peak": HBM / 1e9,
                "unit": "GB/s"}
    else:
        roof = {"bound": "mfma", "achieved": flop / (launch_ms * 1e-3) / 1e12, "peak": peak / 1e12,
                "unit": "TFLOP/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    return roof


def repeats_for(block_ms, minimum, total_ms=50.0):
    """Timed blocks: at least `minimum`, and enough for total_ms in all."""
    return max(minimum, int(math.ceil(total_ms / max(block_ms, 1e-6))))


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def summarize_trace(path, last):
    """Per kernel of a rocprofv3 kernel-trace CSV: launches, and the median,
    min and max duration (ns) of the last `last` launches of it."""
    import csv
    durs = {}
    with open(path, newline="") as f:
        for row in csv.DictReader(f):
            name = row.get("Kernel_Name") or row.get("KernelName") or row.get("Name")
            t0, t1 = int(row["Start_Timestamp"]), int(row["End_Timestamp"])
            durs.setdefault(name, []).append((t0, t1 - t0))
    out = []
    for name, v in durs.items():
        v.sort()
        d = np.array([x[1] for x in v][-last:], dtype=np.float64)
        out.append({"kernel": name, "launches": len(v), "timed": len(d), "median_ns": float(np.median(d)),
                    "min_ns": float(d.min()), "max_ns": float(d.max()), "mean_ns": float(d.mean())})
    return sorted(out, key=lambda e: -e["launches"])


def time_blocks(step, steps, repeats, stream, torch):
    """Milliseconds of each of `repeats` blocks of `steps` launches, each
    block between two events on the launch stream."""
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(repeats)]
    torch.cuda.synchronize()
    i = 0
    for e0, e1 in ev:
        e0.record(stream)
        for _ in range(steps):
            step(i)
            i += 1
        e1.record(stream)
    torch.cuda.synchronize()
    return [e0.elapsed_time(e1) for e0, e1 in ev]


def warm(step, warmup, seconds, torch):
    """W untimed steps, then more until `seconds` of work have run: the
    clocks ramp up under load (after 20 steps alone the next ones ran 15-20 %
    slower than after 0.3 s of work)."""
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    extra = 0
    t_w = time.perf_counter()
    while time.perf_counter() - t_w < seconds:
        for _ in range(20):
            step(warmup + extra)
            extra += 1
        torch.cuda.synchronize()
    return extra


def cpu_baseline(oracle, otype, c, A, Bs, flop, seconds):
    """The oracle as it stands on this host's cores, over a bounded sample of
    the workload's rows (the whole cascade per row), about `seconds` long."""
    nthreads = len(os.sched_getaffinity(0))
    rows_total = c["batch"] * c["M"]
    per_row = flop / rows_total
    n = 2048
    t0 = time.perf_counter()
    oracle.cascade(otype, A, Bs, rows=np.arange(n, dtype=np.int64), nthreads=nthreads)
    dt1 = time.perf_counter() - t0
    n2 = int(min(rows_total, max(n, n * seconds / max(dt1, 1e-6))))
    idx = np.linspace(0, rows_total - 1, n2).astype(np.int64)
    passes, el = 0, 0.0
    # a sample that is the whole workload and ends early is repeated until the target time
    while passes == 0 or (n2 == rows_total and el < seconds):
        t0 = time.perf_counter()
        oracle.cascade(otype, A, Bs, rows=idx, nthreads=nthreads)
        el += time.perf_counter() - t0
        passes += 1
    what = (f"{n2} of {rows_total} rows spread over all batches" if passes == 1 else
            f"{passes} passes over all {n2} rows")
    return {"value": passes * n2 * per_row / el / 1e12, "unit": "TFLOP/s", "cores": nthreads,
            "kind": "oracle", "cpu_model": cpu_model(), "seconds": el,
            "sample": what + ", full cascade per row"}


def measure_ceilings(cf, torch, stream, repeats):
    """Practical ceilings of this device: the matrix cores alone per dtype
    (TFLOP/s) and a copy stream (GB/s of reads plus writes), each the median
    over `repeats` timed launches (the copy over rotating buffer pairs of
    1 GiB in all, so it streams from HBM)."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    wg = 2 * cus                                     # two waves per SIMD
    sink = torch.empty(wg * 256, dtype=torch.float64, device="cuda")
    out = {"workgroups": wg}
    # rounds per launch for ~2 ms at the expected rates
    iters = {"f16": 8192, "bf16": 8192, "f64": 3072}
    mfma = {}
    for dt, it in iters.items():
        flop = cf.bench_mfma(dt, wg, it, sink, stream=stream)
        ms = time_blocks(lambda i: cf.bench_mfma(dt, wg, it, sink, stream=stream), 1, repeats + 1, stream, torch)[1:]
        mfma[dt] = flop / (float(np.median(ms)) * 1e-3) / 1e12
    out["mfma_tflops"] = mfma
    # 128 MiB read + 128 MiB written per launch over four pairs, four
    # workgroups a compute unit: the best of the sizes and grids measured
    nbytes = 128 << 20
    pairs = [(torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1),
              torch.empty(nbytes, dtype=torch.uint8, device="cuda")) for _ in range(4)]
    cwg = 4 * cus

    def copy(i):
        s, d = pairs[i % len(pairs)]
        cf.bench_copy(s, d, cwg, stream=stream)
    copy(0)
    ms = time_blocks(copy, len(pairs), repeats, stream, torch)
    per = float(np.median(ms)) / len(pairs)
    out["copy_gbps"] = 2 * nbytes / (per * 1e-3) / 1e9
    out["copy_bytes"] = nbytes
    del pairs
    return out


def measure_stream(cf, torch, stream, sets, steps, repeats):
    """The workload's own A (read) and D (written) buffers, over the same
    rotating sets, moved by the mixed stream b2b_bench_stream: the time the
    memory system needs for exactly this mix of bytes with nothing else to do,
    the fastest of two and four workgroups a compute unit.  None when A's
    bytes are not 1 to 4 times D's."""
    A0, _, D0 = sets[0]
    rb, wb = A0.numel() * A0.element_size(), D0.numel() * D0.element_size()
    if wb < 64 or wb % 64 or rb % wb or not 1 <= rb // wb <= 4:
        return None
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    best = None
    for per_cu in (2, 4):
        wg = per_cu * cus

        def st(i):
            Ad, _, D = sets[i % len(sets)]
            cf.bench_stream(Ad, D, wg, stream=stream)
        warm(st, 20, 0.1, torch)
        ms = float(np.median(time_blocks(st, steps, repeats, stream, torch))) / steps
        if best is None or ms < best[0]:
            best = (ms, wg)
    ms, wg = best
    return {"ms_per_step": ms, "gbps": (rb + wb) / (ms * 1e-3) / 1e9, "read_bytes": rb, "write_bytes": wb,
            "reads_per_write": rb // wb, "workgroups": wg}


DTYPE_NAMES = {"f16": "fp16", "bf16": "bf16", "f64": "fp64", "tf32": "tf32"}


def measure(cfg_id, args, cf, torch, synth, oracle, cpu_seconds, ceilings=None, log=True):
    """One workload: build the plan and rotating buffer sets, warm up, time
    the blocks, check sampled rows against the oracle, time the oracle."""
    c = dict(synth.WORKLOADS[cfg_id])
    if args.dtype and args.dtype != c["dtype"]:
        # the name leads with the type ("fp16 b16 ..."): the new type's name replaces it
        c["name"] = DTYPE_NAMES[args.dtype] + " " + c["name"].split(" ", 1)[1]
        c["dtype"] = args.dtype
    if args.dims:
        c["dims"] = [int(x) for x in args.dims.split(",")]
        c["name"] = (f"{DTYPE_NAMES[c['dtype']]} b{c['batch']} {c['M']}x{c['dims'][0]} . "
                     + " . ".join(f"{c['dims'][s]}x{c['dims'][s + 1]}" for s in range(len(c["dims"]) - 1)))
    dt = c["dtype"]
    types = args.types.split(",") if args.types else None
    if types:
        c["name"] += " types " + "/".join(types)
    flop, algo_bytes = workload_numbers(c, types)
    if log:
        print(f"[bench] config {cfg_id}: {c['name']}; generating inputs", file=sys.stderr, flush=True)
    A, Bs = synth.make_inputs(c, types=types)
    st_types = types or [dt] * len(c["dims"])
    set_bytes = (A.nbytes + sum(b.nbytes for b in Bs)
                 + c["batch"] * c["M"] * c["dims"][-1] * ELT[st_types[-1]])
    R = max(1, min(64, int(np.ceil(args.rotate_bytes / set_bytes))))
    A0 = cf.to_device(A, st_types[0])
    B0 = [cf.to_device(b, st_types[s]) for s, b in enumerate(Bs)]
    sets = []
    for r in range(R):
        Ad = A0 if r == 0 else A0.clone()
        Bd = B0 if r == 0 else [b.clone() for b in B0]
        D = torch.empty((c["batch"], c["M"], c["dims"][-1]),
                        dtype=cf.TORCH_DTYPES[cf.DTYPES[st_types[-1]]], device="cuda")
        sets.append((Ad, Bd, D))
    dims = c["dims"]
    if types:
        plan = cf.Chain(types, c["batch"], c["M"], dims, remap=args.remap, unfused=args.unfused)
    elif len(dims) <= 4:
        plan = cf.Plan(dt, c["batch"], c["M"], *dims[:3], dims[3] if len(dims) > 3 else 0,
                       remap=args.remap, orient_n=args.orient_n, unfused=args.unfused, mfma32=args.mfma32,
                       tf32_exact=args.tf32_exact)
    else:   # longer cascades: the chain entry points
        plan = cf.Chain(dt, c["batch"], c["M"], dims, remap=args.remap, unfused=args.unfused,
                        mfma32=args.mfma32, tf32_exact=args.tf32_exact)
    stream = torch.cuda.current_stream()
    if args.tune:
        plan.tune(sets, reps=2 * R, stream=stream)
        if log:
            print(f"[bench] tuned: {plan.info()}", file=sys.stderr, flush=True)

    def step(i):
        Ad, Bd, D = sets[i % R]
        plan.run(Ad, *Bd, D=D, stream=stream)

    if args.latency:
        # one launch at a time: event pair around it, wait for it, next launch
        for i in range(max(args.warmup, 20)):
            step(i)
        torch.cuda.synchronize()
        lat = []
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        for i in range(args.latency):
            e0.record(stream)
            step(i)
            e1.record(stream)
            e1.synchronize()
            lat.append(e0.elapsed_time(e1) * 1e3)
        lat = np.array(lat)
        return {"metric": "single-launch latency", "unit": "us", "launches": args.latency,
                "median": float(np.median(lat)), "p10": float(np.percentile(lat, 10)),
                "p90": float(np.percentile(lat, 90)), "min": float(lat.min()),
                "config": {"workload": c["name"], "plan": plan.info()}}

    extra = warm(step, args.warmup, args.warmup_seconds, torch)
    # one untimed block sizes the repeats (at least args.repeats, 50 ms in all)
    est = time_blocks(step, args.steps, 1, stream, torch)[0]
    repeats = repeats_for(est, args.repeats)
    if log:
        print(f"[bench] config {cfg_id}: warmup {args.warmup} + {extra} steps; timing {repeats} x "
              f"{args.steps} steps over {R} buffer sets", file=sys.stderr, flush=True)
    blocks = time_blocks(step, args.steps, repeats, stream, torch)
    per_step = sorted(b / args.steps for b in blocks)
    ms_per_step = float(np.median(per_step))
    launches = int(dict(kv.split("=") for kv in plan.info().split()).get("launches", 1))
    # the fused path is one launch a step: the events around a block bound
    # the back-to-back launches, so the step time is the kernel's duration
    # plus the gap between two launches on the stream
    launch_ms = ms_per_step / launches
    value = flop / (ms_per_step * 1e-3) / 1e12
    pk = PEAK["tf32x4" if args.tf32_exact else dt]
    roof = roofline(flop, algo_bytes, ms_per_step, pk)
    roof["traffic"] = None
    plain = (not args.unfused and args.remap == "auto" and not args.orient_n and not args.mfma32
             and not args.dims and not args.tune and not types and not args.dtype)
    try:
        from chip_fusion_amd import build as _b
        tr = json.load(open(os.path.join(ROOT, "profiles", "traffic.json")))
        ent = tr["configs"].get(str(cfg_id))
        # HBM bytes per launch from the committed rocprofv3 counters, valid
        # only while the kernel sources are the ones they were taken with
        if ent and tr["source_digest"] == _b.source_digest() and plain:
            roof["traffic"] = ent["hbm_bytes"]
            roof["traffic_unit"] = "bytes per launch (FETCH_SIZE x %.3f + WRITE_SIZE x %.3f)" % (
                tr["fetch_scale"], tr["write_scale"])
    except (OSError, ValueError, KeyError):
        pass
    roof["kernel_ms"] = launch_ms
    roof["kernel_ms_min"] = per_step[0] / launches
    roof["kernel_ms_max"] = per_step[-1] / launches
    roof["launches_per_step"] = launches
    roof["algorithmic_bytes"] = algo_bytes
    roof["algorithmic_flop"] = flop
    if ceilings:
        roof["frac_of_measured_copy_bw"] = (algo_bytes / (launch_ms * 1e-3) / 1e9) / ceilings["copy_gbps"]

    # check the last buffer set written against the oracle on a few rows
    rows = np.linspace(0, c["batch"] * c["M"] - 1, 64).astype(np.int64)
    last = (len(blocks) * args.steps - 1) % R
    got = cf.to_host(sets[last][2]).reshape(-1, dims[-1])[rows]
    otype = types if types else dt
    ref = oracle.cascade(otype, A, Bs, rows=rows)
    g, rf = (oracle.decode(st_types[-1], got).astype(np.float64),
             oracle.decode(st_types[-1], ref).astype(np.float64))
    sample_err = float(np.linalg.norm(g - rf) / np.linalg.norm(rf))
    if ceilings:
        # after the check: the stream overwrites D
        sm = measure_stream(cf, torch, stream, sets, args.steps, repeats)
        if sm:
            roof["stream"] = sm
            roof["frac_of_measured_stream"] = sm["ms_per_step"] / launch_ms
    plan_info = plan.info()
    plan.close()
    del sets, A0, B0
    torch.cuda.empty_cache()

    cpu = cpu_baseline(oracle, otype, c, A, Bs, flop, cpu_seconds) if cpu_seconds > 0 else None
    entry = {
        "workload": c["name"],
        "value": value,
        "unit": "TFLOP/s",
        "dtype": "/".join(types) if types else dt,
        "ms_per_step": ms_per_step,
        "ms_per_step_min": per_step[0],
        "ms_per_step_max": per_step[-1],
        "steps": args.steps,
        "repeats": repeats,
        "warmup_extra_steps": extra,
        "pct_of_mfma_peak": 100.0 * value * 1e12 / pk,
        "roofline": roof,
        "cpu_baseline": cpu,
        "sample_rel_err": sample_err,
        "config": {"workload": c["name"], "batch": c["batch"], "M": c["M"], "dims": dims,
                   "path": "unfused" if args.unfused else "fused", "remap": args.remap,
                   "orientation": "N" if args.orient_n else "T", "rotating_buffer_sets": R,
                   "plan": plan_info},
    }
    if ceilings and dt in ceilings["mfma_tflops"]:
        entry["pct_of_measured_mfma_ceiling"] = 100.0 * value / ceilings["mfma_tflops"][dt]
    return entry


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200, help="launches per timed block")
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--repeats", type=int, default=5,
                    help="timed blocks (at least; more until 50 ms in all); the median block counts")
    ap.add_argument("--config", type=int, default=None,
                    help="one workload 1-5; default: the largest of each dtype (5 headline, 3, 4)")
    ap.add_argument("--remap", default="auto")
    ap.add_argument("--orient-n", action="store_true")
    ap.add_argument("--unfused", action="store_true")
    ap.add_argument("--mfma32", action="store_true",
                    help="kernels on the 32x32x16 instruction with run-time widths")
    ap.add_argument("--tune", action="store_true",
                    help="let the library time its candidate kernels on the buffer sets and keep the fastest")
    ap.add_argument("--dims", default=None,
                    help="comma-separated widths K,N1,N2[,N3] replacing the workload's (same batch, M, "
                         "distribution and seed)")
    ap.add_argument("--dtype", default=None, choices=["f16", "bf16", "f64", "tf32"],
                    help="run the workload's shape, distribution and seed in another type")
    ap.add_argument("--tf32-exact", action="store_true", help="tf32 with four bf16 passes per product")
    ap.add_argument("--types", default=None,
                    help="comma-separated 16-bit type per GEMM and one for D (e.g. f16,bf16,f16): "
                         "a cascade with a type per stage on the workload's shape")
    ap.add_argument("--rotate-bytes", type=float, default=1 << 30)
    ap.add_argument("--warmup-seconds", type=float, default=0.3,
                    help="keep warming up (untimed) until this much GPU time has passed, so the "
                         "timed steps run at settled clocks (default 0.3)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="target CPU time of the headline's oracle baseline sample, half of it for "
                         "each further dtype (0 disables)")
    ap.add_argument("--no-ceilings", action="store_true",
                    help="skip the matrix-core and copy-stream ceiling measurements")
    ap.add_argument("--latency", type=int, default=0, metavar="N",
                    help="instead of throughput: N single launches, each timed alone with HIP "
                         "events and a synchronisation in between; prints latency percentiles")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="BYTES",
                    help="only run device-to-device copies of BYTES (scale for HBM counters)")
    ap.add_argument("--summarize-trace", default=None, metavar="CSV",
                    help="only summarise a rocprofv3 kernel trace: per kernel, the last --last launches")
    ap.add_argument("--last", type=int, default=1000)
    args = ap.parse_args()

    if args.summarize_trace:
        for e in summarize_trace(args.summarize_trace, args.last):
            print(json.dumps(e))
        return

    if args.calibrate_copy:
        import torch
        n = args.calibrate_copy
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": n, "copies": args.steps}))
        return

    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(the cascade would shard by rows of A and D, each GPU holding every weight, with no exchange)", file=sys.stderr)
        sys.exit(2)

    if args.tf32_exact and args.dtype != "tf32":
        print("--tf32-exact needs --dtype tf32", file=sys.stderr)
        sys.exit(2)
    if args.types:
        types = args.types.split(",")
        c = synth_workload(args.config or HEADLINE)
        ok = (len(types) == len(args.dims.split(",") if args.dims else c["dims"]) and c["dtype"] != "f64"
              and types[0] != "fp8" and types[-1] != "fp8" and all(t in ("f16", "bf16", "fp8") for t in types))
        if not ok:
            print("--types takes f16/bf16 per GEMM (fp8 for a later one) and f16/bf16 for D, on a 16-bit "
                  "workload", file=sys.stderr)
            sys.exit(2)

    import torch

    import chip_fusion_amd as cf
    import oracle
    import synth

    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    # the per-dtype entries belong to the default run: the largest workload
    # of each dtype, as compiled and planned by default
    single = (args.config is not None or args.dtype or args.dims or args.types or args.unfused or args.mfma32
              or args.tune or args.orient_n or args.remap != "auto")
    cfg = args.config or HEADLINE

    if args.latency:
        print(json.dumps(measure(cfg, args, cf, torch, synth, oracle, 0)))
        return

    ceilings = None
    if not args.no_ceilings:
        print("[bench] ceilings: matrix cores alone, copy stream", file=sys.stderr, flush=True)
        ceilings = measure_ceilings(cf, torch, stream, args.repeats)

    head = measure(cfg, args, cf, torch, synth, oracle, args.cpu_seconds, ceilings)
    dt = head["dtype"]
    out = {
        "metric": "fused B2B-GEMM TFLOP/s per dtype + % of MI355X dense MFMA peak, 1 GPU",
        "value": head["value"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "repeats": head["repeats"],
        "warmup_extra_steps": head["warmup_extra_steps"],
        "ms_per_step": head["ms_per_step"],
        "ms_per_step_min": head["ms_per_step_min"],
        "ms_per_step_max": head["ms_per_step_max"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dt,
        "data": "synthetic",
        "pct_of_mfma_peak": head["pct_of_mfma_peak"],
        "config": head["config"],
        "roofline": head["roofline"],
        "cpu_baseline": head["cpu_baseline"],
        "sample_rel_err": head["sample_rel_err"],
    }
    if "pct_of_measured_mfma_ceiling" in head:
        out["pct_of_measured_mfma_ceiling"] = head["pct_of_measured_mfma_ceiling"]
    if ceilings:
        out["frac_of_measured_copy_bw"] = head["roofline"].get("frac_of_measured_copy_bw")
        out["frac_of_measured_stream"] = head["roofline"].get("frac_of_measured_stream")
        out["ceilings"] = ceilings
    if not single:
        per = {"f16": {k: head[k] for k in head if k != "config"}}
        for d, c_id in PER_DTYPE.items():
            if c_id == cfg:
                continue
            e = measure(c_id, args, cf, torch, synth, oracle, args.cpu_seconds / 2, ceilings)
            e.pop("config")
            per[d] = e
        out["per_dtype"] = per
    print(json.dumps(out))


def synth_workload(cfg):
    import synth
    return synth.WORKLOADS[cfg]


if __name__ == "__main__":
    main()
