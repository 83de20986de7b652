"""Throughput of the fused cascaded GEMM on one MI355X.

A step is one fused cascade D = rnd(rnd(A.B0).B1)[.B2] over one batch of the
workload (one kernel launch).  Inputs are seeded synthetic tensors already in
HBM; the timed loop rotates over enough copies of them (>= 1 GiB in total, four
times the 256 MB Infinity Cache) that every step reads A and writes D in HBM.

Prints one JSON line: TFLOP/s of the whole job, the dominant kernel's
roofline figures (algorithmic bytes or FLOP over its measured duration), and
the CPU oracle timed on a bounded sample of the same workload.
"""
import argparse
import json
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


def workload_numbers(c, types=None):
    """FLOP and algorithmic bytes (A + weights + D) of a step; types: one per
    GEMM and D's, when the stages differ."""
    dims, b, M = c["dims"], c["batch"], c["M"]
    t = types or [c["dtype"]] * len(dims)
    flop = 2.0 * b * M * sum(dims[s] * dims[s + 1] for s in range(len(dims) - 1))
    wbytes = b * sum(dims[s] * dims[s + 1] * ELT[t[s]] for s in range(len(dims) - 1))
    byts = b * M * dims[0] * ELT[t[0]] + wbytes + b * M * dims[-1] * ELT[t[-1]]
    return flop, byts


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=2, help="workload 1-5 (default 2)")
    ap.add_argument("--remap", default="auto")
    ap.add_argument("--orient-n", action="store_true")
    ap.add_argument("--unfused", action="store_true")
    ap.add_argument("--mfma32", action="store_true",
                    help="kernels on the 32x32x16 instruction with run-time widths")
    ap.add_argument("--tune", action="store_true",
                    help="let the library time its candidate kernels on the first buffer set and keep the fastest")
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
                    help="target CPU time of the oracle baseline sample (0 disables)")
    ap.add_argument("--latency", type=int, default=0, metavar="N",
                    help="instead of throughput: N single launches, each timed alone with HIP "
                         "events and a synchronisation in between; prints latency percentiles")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="BYTES",
                    help="only run device-to-device copies of BYTES (scale for HBM counters)")
    args = ap.parse_args()

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
              "(the cascade shards by rows with no exchange; see the design notes)", file=sys.stderr)
        sys.exit(2)

    import torch

    import chip_fusion_amd as cf
    import synth

    c = dict(synth.WORKLOADS[args.config])
    if args.dtype and args.dtype != c["dtype"]:
        c["name"] = c["name"].replace(c["dtype"], args.dtype, 1)
        c["dtype"] = args.dtype
    if args.tf32_exact and c["dtype"] != "tf32":
        print("--tf32-exact needs --dtype tf32", file=sys.stderr)
        sys.exit(2)
    if args.dims:
        c["dims"] = [int(x) for x in args.dims.split(",")]
        c["name"] = (f"{c['dtype']} b{c['batch']} {c['M']}x{c['dims'][0]} . "
                     + " . ".join(f"{c['dims'][s]}x{c['dims'][s + 1]}" for s in range(len(c["dims"]) - 1)))
    dt = c["dtype"]
    types = args.types.split(",") if args.types else None
    if types:
        ok = (len(types) == len(c["dims"]) and dt != "f64" and types[0] != "fp8" and types[-1] != "fp8"
              and all(t in ("f16", "bf16", "fp8") for t in types))
        if not ok:
            print("--types takes f16/bf16 per GEMM (fp8 for a later one) and f16/bf16 for D, on a 16-bit "
                  "workload", file=sys.stderr)
            sys.exit(2)
        c["name"] += " types " + "/".join(types)
    flop, algo_bytes = workload_numbers(c, types)
    print(f"[bench] config {args.config}: {c['name']}; generating inputs", file=sys.stderr, flush=True)
    A, Bs = synth.make_inputs(c, types=types)
    st_types = types or [dt] * len(c["dims"])
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    set_bytes = A.nbytes + sum(b.nbytes for b in Bs) + c["batch"] * c["M"] * c["dims"][-1] * ELT[(types or [dt])[-1]]
    R = max(1, min(64, int(np.ceil(args.rotate_bytes / set_bytes))))
    A0 = cf.to_device(A, st_types[0])
    B0 = [cf.to_device(b, st_types[s]) for s, b in enumerate(Bs)]
    sets = []
    for r in range(R):
        Ad = A0 if r == 0 else A0.clone()
        Bd = B0 if r == 0 else [b.clone() for b in B0]
        D = torch.empty((c["batch"], c["M"], c["dims"][-1]), dtype=cf.TORCH_DTYPES[cf.DTYPES[st_types[-1]]],
                        device=dev)
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
        print(json.dumps({"metric": "single-launch latency", "unit": "us", "launches": args.latency,
                          "median": float(np.median(lat)), "p10": float(np.percentile(lat, 10)),
                          "p90": float(np.percentile(lat, 90)), "min": float(lat.min()),
                          "config": {"workload": c["name"], "plan": plan.info()}}))
        return

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    # The GPU's clocks ramp up under sustained load: a short warmup leaves the
    # first timed steps at lower clocks (measured: 15-20 % slower per step
    # after 20 warmup steps than after 0.3 s of work).  Warm up further, in
    # untimed steps, until warmup_seconds of work have passed.
    extra = 0
    t_w = time.perf_counter()
    while time.perf_counter() - t_w < args.warmup_seconds:
        for _ in range(20):
            step(args.warmup + extra)
            extra += 1
        torch.cuda.synchronize()
    print(f"[bench] warmup done ({args.warmup} + {extra} steps); timing {args.steps} steps over {R} "
          "buffer sets", file=sys.stderr, flush=True)

    # whole timed region
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for i in range(args.steps):
        step(i)
    t_end.record(stream)
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    ms_per_step = total_ms / args.steps

    # Duration of the launch(es) of one step, from the events around the timed
    # region on the stream the kernels run on.  Bracketing each launch with its
    # own events instead adds the event packets' gaps (about 3 us a launch).
    # Where a run is more than one launch (the column-split path packs its
    # weights first), this is the whole step, so the roofline figure below
    # understates the fused kernel alone.
    launch_ms = ms_per_step
    launches = int(dict(kv.split("=") for kv in plan.info().split()).get("launches", 1))

    value = flop / (ms_per_step * 1e-3) / 1e12
    ai = flop / algo_bytes
    pk = PEAK["tf32x4" if args.tf32_exact else dt]
    ridge = pk / HBM
    if ai < ridge:
        roof = {"bound": "hbm", "achieved": algo_bytes / (launch_ms * 1e-3) / 1e9, "peak": HBM / 1e9,
                "unit": "GB/s"}
    else:
        roof = {"bound": "mfma", "achieved": flop / (launch_ms * 1e-3) / 1e12, "peak": pk / 1e12,
                "unit": "TFLOP/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    # HBM bytes per launch from the committed rocprofv3 counters, valid only
    # while the kernel sources are the ones they were taken with
    roof["traffic"] = None
    try:
        from chip_fusion_amd import build as _b
        tr = json.load(open(os.path.join(ROOT, "profiles", "traffic.json")))
        ent = tr["configs"].get(str(args.config))
        if (ent and tr["source_digest"] == _b.source_digest() and not args.unfused
                and args.remap == "auto" and not args.orient_n and not args.mfma32 and not args.dims
                and not args.tune and not types and not args.dtype):
            roof["traffic"] = ent["hbm_bytes"]
            roof["traffic_unit"] = "bytes per launch (FETCH_SIZE x %.3f + WRITE_SIZE x %.3f)" % (
                tr["fetch_scale"], tr["write_scale"])
    except (OSError, ValueError, KeyError):
        pass
    roof["kernel_ms"] = launch_ms
    roof["launches_per_step"] = launches
    roof["algorithmic_bytes"] = algo_bytes
    roof["algorithmic_flop"] = flop

    # check the last buffer set against the oracle on a few rows (cheap sanity)
    import oracle
    rows = np.linspace(0, c["batch"] * c["M"] - 1, 64).astype(np.int64)
    got = cf.to_host(sets[(args.steps - 1) % R][2]).reshape(-1, dims[-1])[rows]
    otype = types if types else dt
    ref = oracle.cascade(otype, A, Bs, rows=rows)
    g, rf = (oracle.decode(st_types[-1], got).astype(np.float64),
             oracle.decode(st_types[-1], ref).astype(np.float64))
    sample_err = float(np.linalg.norm(g - rf) / np.linalg.norm(rf))

    cpu = None
    if args.cpu_seconds > 0:
        nthreads = len(os.sched_getaffinity(0))
        per_row = flop / (c["batch"] * c["M"])
        n = 2048
        t0 = time.perf_counter()
        oracle.cascade(otype, A, Bs, rows=np.arange(n, dtype=np.int64), nthreads=nthreads)
        dt1 = time.perf_counter() - t0
        n2 = int(min(c["batch"] * c["M"], max(n, n * args.cpu_seconds / max(dt1, 1e-6))))
        idx = np.linspace(0, c["batch"] * c["M"] - 1, n2).astype(np.int64)
        # a sample that is the whole workload and ends early is repeated until the target time
        passes, el = 0, 0.0
        while passes == 0 or (n2 == c["batch"] * c["M"] and el < args.cpu_seconds):
            t0 = time.perf_counter()
            oracle.cascade(otype, A, Bs, rows=idx, nthreads=nthreads)
            el += time.perf_counter() - t0
            passes += 1
        what = (f"{n2} of {c['batch'] * c['M']} rows spread over all batches" if passes == 1 else
                f"{passes} passes over all {n2} rows")
        cpu = {"value": passes * n2 * per_row / el / 1e12, "unit": "TFLOP/s", "cores": nthreads,
               "kind": "oracle", "seconds": el, "sample": what + ", full cascade per row"}

    out = {
        "metric": "fused B2B-GEMM TFLOP/s (" + dt + ") + % of MI355X dense MFMA peak, 1 GPU",
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_extra_steps": extra,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "/".join(types) if types else dt,
        "data": "synthetic",
        "pct_of_mfma_peak": 100.0 * value * 1e12 / pk,
        "config": {"workload": c["name"], "batch": c["batch"], "M": c["M"], "dims": dims,
                   "path": "unfused" if args.unfused else "fused", "remap": args.remap,
                   "orientation": "N" if args.orient_n else "T", "rotating_buffer_sets": R,
                   "plan": plan.info()},
        "roofline": roof,
        "cpu_baseline": cpu,
        "sample_rel_err": sample_err,
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
