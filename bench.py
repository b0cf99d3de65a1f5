"""Benchmark the dense projection hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload IDX]

A step is one projection Y = epi(X . W^T + bias) over one batch of synthetic
input (one proj_run: plan lookup, kernel, fused epilogue), replayed from a
HIP graph captured through the library (proj_graph_capture).  Steps cycle
over P rotating buffer sets (distinct allocations of X, W, bias, Y) whose
total size exceeds the 256 MiB last-level cache, so W streams from HBM as it
would in a model.  Inputs are resident in HBM before the timed region.

Timing: HIP events recorded on the stream the graph is launched on, around
exactly K steps, with device synchronisation on both sides.  The dominant
(only) kernel of a step is the projection kernel; its average duration is
taken as the timed region divided by K (this includes the small gaps between
graph nodes, so it is an upper bound on the kernel's own duration).

Prints ONE JSON line.  Default workload: M=16 K=8192 N=8192, bias, bf16 out.
Beside the row-major figure the line carries the same steps with W
registered in the packed tile layout (`packed_weights`), five repeat trials,
a cache-resident (warm) figure, the oracle's CPU rate and the device, and
under `workloads` the other four workloads, each set up and timed the same
way in the same process (time per call, roofline against its own bound,
plan; --no-workloads skips them).

Other modes: --sweep (the thirty-shape set, torch timed alongside),
--candidate NAME (one plan repeated, for counter passes), --copy-calibration
and --ingest (scaling and storing rocprofv3 traffic counters).
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "TFLOP/s + achieved HBM GB/s (% roofline) for bf16 Y=X·Wᵀ, M=16 K=8192"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, published
LLC_BYTES = 256 << 20          # last-level (Infinity) cache


# the source files that define each kernel family (the counters of a family
# are stale once any of its files changes)
FAMILY_SOURCES = {
    "stream_kernel": ["stream.hip", "common.hpp"],
    "gemm_pp_kernel": ["gemm.hip", "common.hpp"],
    "gemm_pp64_kernel": ["gemm.hip", "common.hpp"],
    "gemm_pp64p_kernel": ["gemm.hip", "common.hpp"],
    "gemm_kernel": ["gemm.hip", "common.hpp"],
    "gemv_kernel": ["gemv.hip", "common.hpp"],
}


def kernel_sources_hash(family: str) -> str:
    h = hashlib.sha256()
    for name in FAMILY_SOURCES[family]:
        with open(os.path.join(ROOT, "dense_linear_projection_amd", "csrc", name), "rb") as f:
            h.update(name.encode())
            h.update(f.read())
    return h.hexdigest()[:16]


def counters_path(workload_name: str) -> str:
    return os.path.join(ROOT, "profiles", "counters_%s.json" % workload_name)


def load_traffic(workload_name: str, plan_kernel: str):
    """HBM bytes per launch of the planned (dominant) kernel, from committed
    rocprofv3 counter runs (FETCH_SIZE and WRITE_SIZE, each scaled by what
    the same counter reads for a plain copy of known size), if they were
    taken on the current sources of that kernel's family and include this
    plan; else None."""
    path = counters_path(workload_name)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        c = json.load(f)
    entry = c.get("plans", {}).get(plan_kernel)
    if entry is None or entry.get("src_hash") != kernel_sources_hash(entry["family"]):
        return None
    return round(entry["traffic_bytes_per_launch"], 1)


def plan_launch(plan: str, w, cus: int = 256):
    """(family, kernel-name part, work-items) of the dominant kernel a plan
    launches on workload w: the streaming kernel of a stream plan (split or
    not, atomic or not; the zero fill or split-K pass beside it is small), or
    the GEMM kernel, e.g. stream_mt1_nt2_w4_k128_d4_wnt_s1 ->
    ("stream_kernel", "stream_kernel<1, 2, 4, 128, 4, 1, true>", 65536)."""
    import re
    m = re.fullmatch(r"stream_mt(\d+)_nt(\d+)_w(\d+)_k(\d+)_d(\d+)(_wnt)?_s(\d+)(_atomic)?(_r\d+)?", plan)
    if m is not None:
        mt, nt, waves, kc, d = (int(m.group(i)) for i in range(1, 6))
        wnt, S = m.group(6) is not None, int(m.group(7))
        fast = w.K % kc == 0  # whole stages take the buffer-resource copy path
        name = "stream_kernel<%d, %d, %d, %d, %d, %d, %s>" % (mt, nt, waves, kc, d, int(wnt),
                                                              "true" if fast else "false")
        tiles = -(-w.N // (16 * nt))
        mblocks = -(-w.M // (16 * mt))
        return "stream_kernel", name, mblocks * tiles * S * waves * 64
    m = re.fullmatch(r"gemmpp64([pd]?)_256x(\d+)x64_w4x2_g(\d+)(_s(\d+))?", plan)
    if m is not None:
        kind, bn, gm = m.group(1), int(m.group(2)), int(m.group(3))
        S = int(m.group(5) or 1)
        G = -(-w.M // 256) * -(-w.N // bn) * S
        if kind == "":
            return "gemm_pp64_kernel", "gemm_pp64_kernel<%d, %d>" % (bn, gm), G * 512
        return ("gemm_pp64p_kernel", "gemm_pp64p_kernel<%d, %d, %s>" % (bn, gm, "true" if kind == "d" else "false"),
                min(G, cus) * 512)
    raise SystemExit("no counter mapping for plan %r" % plan)


def _pmc_per_dispatch(run_dir: str, counter: str, name_part: str, skip_first: int = 0, grid: int = 0):
    """Mean of one counter over the dispatches of kernels whose name holds
    name_part (and, if grid > 0, whose grid has that many work-items), from a
    rocprofv3 --pmc CSV output directory."""
    import csv
    vals = {}
    for path in glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True):
        with open(path) as f:
            for r in csv.DictReader(f):
                if grid and int(r["Grid_Size"]) != grid:
                    continue
                if name_part in r["Kernel_Name"] and r["Counter_Name"] == counter:
                    key = (path, r["Dispatch_Id"])
                    vals[key] = vals.get(key, 0.0) + float(r["Counter_Value"])
    xs = [v for _, v in sorted(vals.items(), key=lambda kv: int(kv[0][1]))][skip_first:]
    if not xs:
        raise SystemExit("no %s samples for kernels matching %r in %s" % (counter, name_part, run_dir))
    return sum(xs) / len(xs), len(xs)


def ingest_counters(args) -> int:
    """Write profiles/counters_<workload>.json from four rocprofv3 --pmc runs:
    FETCH_SIZE and WRITE_SIZE of this bench, and of --copy-calibration.  The
    plan tuner runs every candidate on cold caches, so one pair of runs holds
    samples of each candidate plan; each plan named in --plans gets its own
    figures, taken on its own kernel instantiation and grid."""
    import synth
    w = synth.WORKLOADS[args.workload]
    cfetch, _ = _pmc_per_dispatch(args.ingest[2], "FETCH_SIZE", "copy")
    cwrite, _ = _pmc_per_dispatch(args.ingest[3], "WRITE_SIZE", "copy")
    copy_bytes = COPY_BYTES
    fetch_scale, write_scale = copy_bytes / (cfetch * 1024), copy_bytes / (cwrite * 1024)
    plans = {}
    for plan in args.plans:
        fam, kern, grid = plan_launch(plan, w)
        fetch, nf = _pmc_per_dispatch(args.ingest[0], "FETCH_SIZE", kern, grid=grid)
        write, nw = _pmc_per_dispatch(args.ingest[1], "WRITE_SIZE", kern, grid=grid)
        traffic = fetch * 1024 * fetch_scale + write * 1024 * write_scale
        plans[plan] = {"family": fam, "src_files": FAMILY_SOURCES[fam], "src_hash": kernel_sources_hash(fam),
                       "kernel_name_part": kern, "grid_work_items": grid,
                       "fetch_kib_per_dispatch": fetch, "write_kib_per_dispatch": write,
                       "dispatches": [nf, nw], "traffic_bytes_per_launch": traffic,
                       "traffic_over_alg": traffic / w.alg_bytes()}
    # plans ingested earlier (other counter runs of the same workload) stay
    path = counters_path(w.name)
    if os.path.exists(path):
        with open(path) as f:
            old = json.load(f).get("plans", {})
        plans = {**{k: v for k, v in old.items() if "family" in v}, **plans}
    out = {
        "workload": w.name,
        "copy_bytes": copy_bytes,
        "copy_fetch_kib": cfetch, "copy_write_kib": cwrite,
        "fetch_scale": fetch_scale, "write_scale": write_scale,
        "alg_bytes_per_launch": w.alg_bytes(),
        "plans": plans,
    }
    with open(counters_path(w.name), "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out))
    return 0


def timeline(args) -> int:
    """Per-call timeline of graph-replayed steps from a rocprofv3
    --kernel-trace CSV (run_kernel_trace.csv): the kernels of each call of
    the projection in launch order, their durations and the gaps between
    them and to the next call, as medians over the calls that were replayed
    back to back (a call follows the previous one within --gap-us).  The
    calls are the dispatches of kernels whose name contains one of
    --kernels, grouped so that each group starts with the first of those
    names.  The same kernel may also run for other workloads in the same
    process: --grid NAME_PART:WORK_ITEMS keeps, of the kernels whose name
    contains NAME_PART, only the dispatches of that grid size, and
    --near-us keeps only calls whose kernels span within a factor of 2 of
    that many microseconds."""
    import csv
    grids = []
    for g in args.grid:
        part, items = g.rsplit(":", 1)
        grids.append((part, int(items)))
    rows = []
    with open(args.timeline) as f:
        for r in csv.DictReader(f):
            name = r["Kernel_Name"]
            if not any(k in name for k in args.kernels):
                continue
            size = int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"])
            if any(part in name and size != items for part, items in grids):
                continue
            rows.append((int(r["Start_Timestamp"]), int(r["End_Timestamp"]), name))
    rows.sort()
    first = args.kernels[0]
    calls, cur = [], []
    for r in rows:
        if first in r[2] and cur:
            calls.append(cur)
            cur = []
        cur.append(r)
    if cur:
        calls.append(cur)
    # a call launches each of --kernels once
    n = len(args.kernels)
    steady = []
    for i in range(1, len(calls) - 1):
        c, nxt, prev = calls[i], calls[i + 1], calls[i - 1]
        if len(c) != n or (c[0][0] - prev[-1][1]) > args.gap_us * 1e3 or (nxt[0][0] - c[-1][1]) > args.gap_us * 1e3:
            continue
        # --near-us: only calls whose kernels span within a factor of 2 of
        # it (other workloads' calls of the same kernel and grid differ)
        span = (c[-1][1] - c[0][0]) / 1e3
        if args.near_us > 0 and not (args.near_us / 2 <= span <= 2 * args.near_us):
            continue
        steady.append((c, nxt[0][0]))
    if not steady:
        print("no back-to-back calls found", file=sys.stderr)
        return 1

    def med(xs):
        xs = sorted(xs)
        return xs[len(xs) // 2]
    parts = []
    for j in range(n):
        parts.append({"kernel": steady[0][0][j][2][:90],
                      "duration_us": round(med([c[j][1] - c[j][0] for c, _ in steady]) / 1e3, 3)})
        if j + 1 < n:
            parts.append({"gap_us": round(med([c[j + 1][0] - c[j][1] for c, _ in steady]) / 1e3, 3)})
    parts.append({"gap_to_next_call_us": round(med([t - c[-1][1] for c, t in steady]) / 1e3, 3)})
    per_call = med([t - c[0][0] for c, t in steady]) / 1e3
    print(json.dumps({"calls": len(steady), "kernels_per_call": n, "per_call_us": round(per_call, 3),
                      "timeline": parts}))
    return 0


COPY_BYTES = 256 << 20


def copy_calibration() -> int:
    """A plain device-to-device copy of COPY_BYTES, repeated, for scaling
    the FETCH_SIZE / WRITE_SIZE counters (run under rocprofv3 --pmc)."""
    import torch
    src = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(10):
        dst.copy_(src)
    torch.cuda.synchronize()
    print("copied %d bytes 10 times" % COPY_BYTES)
    return 0


def cpu_baseline(w, X, W, b, min_seconds: float):
    """The oracle as it stands, on the host cores: repeat the whole workload
    (or a fixed slice of its rows for big ones) until min_seconds pass."""
    import numpy as np
    import oracle
    cores = oracle.default_threads()
    # rows of Y in the sample: all rows when the workload is small enough
    macs_per_row = w.N * w.K
    rows = w.M if w.M * macs_per_row <= 4e9 else max(1, int(2e9 // macs_per_row))
    Xs = np.ascontiguousarray(X[:rows])
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.proj_f64(Xs, W, b, w.epi, nthreads=cores)
        reps += 1
        el = time.perf_counter() - t0
        if el >= min_seconds:
            break
    frac = rows / w.M
    bytes_done = w.alg_bytes() * frac * reps
    # one thread, on one row of Y (all N columns, full K), three runs: median
    t1 = []
    for _ in range(3):
        t = time.perf_counter()
        oracle.proj_f64(np.ascontiguousarray(X[:1]), W, b, w.epi, nthreads=1)
        t1.append(time.perf_counter() - t)
    t1.sort()
    one = {"gflops": round(2 * w.N * w.K / t1[1] / 1e9, 3), "seconds_per_row": round(t1[1], 4),
           "sample": "1 row of Y, median of 3"}
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            model = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), "")
    except OSError:
        pass
    return {
        "value": round(bytes_done / el / 1e9, 3),
        "unit": "GB/s",
        "tflops": round(w.alg_flops() * frac * reps / el / 1e12, 6),
        "cores": cores,
        "host_cpus": os.cpu_count(),
        "cpu_model": model,
        "kind": "oracle",
        "sample": "%d of %d rows of Y (all N columns, full K), %d repetition(s), %.1f s, fp64 C oracle"
                  % (rows, w.M, reps, el),
        "single_thread": one,
    }


def sweep_router(sh, ctx, stream, time_replays, to_dev) -> dict:
    """One fp32-weight router shape of the sweep: the weights registered once
    as a bf16 high/low pair (proj_prepare_hilo, outside the timed region),
    then proj_run_hilo calls over rotating buffer sets replayed from a torch
    CUDA graph; torch's fp32 matmul (X converted to fp32 beforehand) is timed
    the same way as context."""
    import numpy as np
    import torch

    import dense_linear_projection_amd as dlp
    import synth

    dev = torch.device("cuda:0")
    X0, W0 = synth.sweep_inputs(sh)
    P = min(16, max(1, -(-(2 * LLC_BYTES) // sh.alg_bytes())))
    R = max(P, 64 // P * P)
    Xs = [to_dev(X0)] + [to_dev(synth.sweep_inputs(sh, 100 * p)[0]) for p in range(1, P)]
    W32 = torch.from_numpy(W0).to(dev)
    Whl0 = dlp.proj_prepare_hilo(ctx, W32, stream=stream)
    Whls = [Whl0] + [Whl0.clone() for _ in range(1, P)]
    Ys = [torch.empty((sh.M, sh.N), dtype=torch.float32, device=dev) for _ in range(P)]
    with torch.cuda.stream(stream):
        for p in range(P):
            dlp.proj_run_hilo(ctx, Xs[p], Whls[p], None, dlp.EPI_NONE, Ys[p], stream=stream)
    stream.synchronize()
    plan = dlp.proj_get_plan_hilo(ctx, sh.M, sh.N, sh.K, dlp.EPI_NONE, synth.OUT_F32)
    idx = [i % P for i in range(R)]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for i in idx:
            dlp.proj_run_hilo(ctx, Xs[i], Whls[i], None, dlp.EPI_NONE, Ys[i], stream=stream)

    def replay_ours():
        with torch.cuda.stream(stream):
            g.replay()

    us = time_replays(replay_ours, R)
    Xf = [x.float() for x in Xs]
    Ws = [W32] + [W32.clone() for _ in range(1, P)]
    Yt = [torch.empty_like(y) for y in Ys]
    with torch.cuda.stream(stream):
        for p in range(P):
            torch.matmul(Xf[p], Ws[p].t(), out=Yt[p])
    stream.synchronize()
    tg = torch.cuda.CUDAGraph()
    with torch.cuda.graph(tg, stream=stream):
        for i in idx:
            torch.matmul(Xf[i], Ws[i].t(), out=Yt[i])

    def replay_torch():
        with torch.cuda.stream(stream):
            tg.replay()

    torch_us = time_replays(replay_torch, R)
    stream.synchronize()
    # the two routes agree to the router's tolerance (both near the fp64 product)
    d = (Ys[0].double() - Yt[0].double()).norm() / Yt[0].double().norm()
    del g, tg
    sec = us * 1e-6
    return {"plan": plan.split(" ")[0], "us": round(us, 3),
            "gbs": round(sh.alg_bytes() / sec / 1e9, 1),
            "hbm_frac": round(sh.alg_bytes() / sec / 1e9 / HBM_PEAK_GBS, 4),
            "tflops": round(sh.alg_flops() / sec / 1e12, 2),
            "torch_us": round(torch_us, 3), "torch_over_ours": round(torch_us / us, 4),
            "rel_l2_vs_torch_fp32": float(d)}


def sweep(args) -> int:
    """The worklog's thirty-shape set (synth.sweep_shapes): for every shape,
    the tuned plan replayed from a HIP graph over rotating buffer sets (the
    main bench's protocol), and beside it torch's matmul (hipBLASLt) replayed
    from a torch CUDA graph the same way -- context, not a target.  Per load
    the five shapes' times are summed; the loads' torch/ours ratios are
    combined by geometric mean, as the worklog scores (section "A quick guide
    to the numbers I'll be showing").  Prints one JSON line."""
    import math
    import numpy as np
    import torch

    import dense_linear_projection_amd as dlp
    import synth

    if not os.path.exists(dlp.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    ctx = dlp.proj_create(0)
    stream = torch.cuda.Stream()
    to_dev = lambda a: torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
    steps = args.sweep_steps
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)

    def time_replays(launch, R):
        for _ in range(3):
            launch()
        stream.synchronize()
        reps = max(1, steps // R)
        e0.record(stream)
        for _ in range(reps):
            launch()
        e1.record(stream)
        e1.synchronize()
        return e0.elapsed_time(e1) * 1e3 / (reps * R)

    rows = []
    for sh in synth.sweep_shapes():
        row = {"name": sh.name, "family": sh.family, "M": sh.M, "N": sh.N, "K": sh.K}
        if sh.fp32_weights:
            row.update(sweep_router(sh, ctx, stream, time_replays, to_dev))
            rows.append(row)
            print(json.dumps(row), file=sys.stderr, flush=True)
            torch.cuda.empty_cache()
            continue
        X0, W0 = synth.sweep_inputs(sh)
        set_bytes = sh.alg_bytes()
        P = min(16, max(1, -(-(2 * LLC_BYTES) // set_bytes)))
        R = max(P, 64 // P * P)
        Xs = [to_dev(X0)] + [to_dev(synth.sweep_inputs(sh, 100 * p)[0]) for p in range(1, P)]
        Wd = to_dev(W0)
        Ws = [Wd] + [Wd.clone() for _ in range(1, P)]
        Ys = [torch.empty((sh.M, sh.N), dtype=torch.bfloat16, device=dev) for _ in range(P)]
        with torch.cuda.stream(stream):
            for p in range(P):
                dlp.proj_run(ctx, Xs[p], Ws[p], None, dlp.EPI_NONE, Ys[p], stream=stream)
        stream.synchronize()
        plan = dlp.proj_get_plan(ctx, sh.M, sh.N, sh.K, dlp.EPI_NONE, synth.OUT_BF16)
        idx = [i % P for i in range(R)]
        g = dlp.proj_graph_capture(ctx, [Xs[i] for i in idx], [Ws[i] for i in idx], None, [Ys[i] for i in idx],
                                   dlp.EPI_NONE, stream=stream)
        us = time_replays(lambda: dlp.proj_graph_launch(g, stream=stream), R)
        dlp.proj_graph_destroy(g)
        # torch: the same products into separate outputs, captured once
        Yt = [torch.empty_like(y) for y in Ys]
        with torch.cuda.stream(stream):
            for p in range(P):
                torch.matmul(Xs[p], Ws[p].t(), out=Yt[p])
        stream.synchronize()
        ref = Yt[0].clone()
        tg = torch.cuda.CUDAGraph()
        with torch.cuda.graph(tg, stream=stream):
            for i in idx:
                torch.matmul(Xs[i], Ws[i].t(), out=Yt[i])
        def replay_on_stream():
            with torch.cuda.stream(stream):
                tg.replay()

        torch_us = time_replays(replay_on_stream, R)
        stream.synchronize()
        torch_ok = bool(torch.equal(Yt[0], ref))
        del tg
        sec = us * 1e-6
        row.update({"plan": plan.split(" ")[0], "us": round(us, 3),
                    "gbs": round(sh.alg_bytes() / sec / 1e9, 1),
                    "hbm_frac": round(sh.alg_bytes() / sec / 1e9 / HBM_PEAK_GBS, 4),
                    "tflops": round(sh.alg_flops() / sec / 1e12, 2),
                    "torch_us": round(torch_us, 3), "torch_replay_matches_eager": torch_ok,
                    "torch_over_ours": round(torch_us / us, 4)})
        rows.append(row)
        print(json.dumps(row), file=sys.stderr, flush=True)
        del Xs, Ws, Ys, Yt, Wd
        torch.cuda.empty_cache()
    dlp.proj_destroy(ctx)

    loads = []
    for M in synth.SWEEP_LOADS:
        rs = [r for r in rows if r["M"] == M and "us" in r]
        ours, theirs = sum(r["us"] for r in rs), sum(r["torch_us"] for r in rs)
        loads.append({"M": M, "shapes_timed": len(rs), "us_sum": round(ours, 3), "torch_us_sum": round(theirs, 3),
                      "torch_over_ours": round(theirs / ours, 4)})
    geo = math.exp(sum(math.log(l["torch_over_ours"]) for l in loads) / len(loads))
    print(json.dumps({"metric": "thirty-shape sweep: per-load time, torch (hipBLASLt) time over ours",
                      "shapes": rows, "loads": loads, "geomean_torch_over_ours": round(geo, 4),
                      "note": "router rows: ours is the bf16 high/low pair (registered outside the timed "
                              "region), torch is an fp32 matmul with X already converted to fp32"}),
          flush=True)
    return 0


def time_packed(ctx, w, args, Xs, Ws, bs, Ys, idx, stream) -> dict:
    """The same steps with W registered once in the packed tile layout
    (proj_pack_weights, outside the timed region), run by proj_run_packed;
    the R calls are captured in a torch CUDA graph (the library's own graph
    helper takes row-major weights)."""
    import torch

    import dense_linear_projection_amd as dlp

    t16, P, R = args.packed, len(Xs), len(idx)
    Wps = [dlp.proj_pack_weights(ctx, Ws[p], t16, stream=stream) for p in range(P)]
    with torch.cuda.stream(stream):
        for p in range(P):                       # plan tuning happens on the first call
            dlp.proj_run_packed(ctx, Xs[p], Wps[p], t16, bs[p], w.epi, Ys[p], w.N, stream=stream)
    stream.synchronize()
    plan = dlp.proj_get_plan_packed(ctx, w.M, w.N, w.K, t16, w.epi, w.out_dtype)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for i in idx:
            dlp.proj_run_packed(ctx, Xs[i], Wps[i], t16, bs[i], w.epi, Ys[i], w.N, stream=stream)
    reps = max(1, args.steps // R)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        for _ in range(max(1, args.warmup // R)):
            g.replay()
        stream.synchronize()
        trial_us = []
        for _ in range(5):
            e0.record(stream)
            for _ in range(reps):
                g.replay()
            e1.record(stream)
            e1.synchronize()
            trial_us.append(e0.elapsed_time(e1) * 1e3 / (reps * R))
    del g
    trial_us.sort()
    us = trial_us[0 + len(trial_us) // 2]
    sec = us * 1e-6
    return {"tile16": t16, "plan": plan, "median_us": round(us, 3), "min_us": round(trial_us[0], 3),
            "max_us": round(trial_us[-1], 3), "gbs": round(w.alg_bytes() / sec / 1e9, 1),
            "tflops": round(w.alg_flops() / sec / 1e12, 2),
            "note": "W packed once before timing (registration); five trials of the same steps, median"}


def time_read_floor(ctx, Ws, idx, stream, args) -> dict:
    """A plain streaming read of the same weight buffers, in the same
    rotation, captured and replayed the same way as the projection: the
    measured floor the weight-streaming kernel is compared with."""
    import torch

    import dense_linear_projection_amd as dlp

    R = len(idx)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for i in idx:
            dlp.proj_read_probe(ctx, Ws[i], stream=stream)
    reps = max(1, args.steps // R)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        g.replay()
        stream.synchronize()
        trial_us = []
        for _ in range(5):
            e0.record(stream)
            for _ in range(reps):
                g.replay()
            e1.record(stream)
            e1.synchronize()
            trial_us.append(e0.elapsed_time(e1) * 1e3 / (reps * R))
    del g
    trial_us.sort()
    us = trial_us[len(trial_us) // 2]
    nbytes = Ws[0].numel() * Ws[0].element_size()
    return {"kernel": "read_probe_kernel", "bytes": nbytes, "median_us": round(us, 3),
            "gbs": round(nbytes / (us * 1e-6) / 1e9, 1),
            "note": "plain streaming read of each W buffer (contiguous slabs, non-temporal 16-byte loads), "
                    "same rotation and graph replay as the projection"}


def run_candidate(args) -> int:
    """Run one candidate plan of a workload args.reps times over two
    buffer sets (no tuning), for rocprofv3 counter passes."""
    import numpy as np
    import torch

    import dense_linear_projection_amd as dlp
    import synth

    w = synth.WORKLOADS[args.workload]
    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    to_dev = lambda a: torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
    names = [dlp.proj_candidate_name(w.M, w.N, w.K, w.epi, w.out_dtype, i)
             for i in range(dlp.proj_num_candidates(w.M, w.N, w.K, w.epi, w.out_dtype))]
    hits = [i for i, n in enumerate(names) if n == args.candidate] or \
        [i for i, n in enumerate(names) if args.candidate in n]
    if not hits:
        print("no candidate contains %r" % args.candidate, file=sys.stderr)
        return 2
    i = hits[0]
    sets = []
    for p in range(2):
        X, W, b = synth.workload_inputs(w, offset=100 * p)
        out_t = torch.float32 if w.out_dtype == synth.OUT_F32 else torch.bfloat16
        sets.append((to_dev(X), to_dev(W), to_dev(b) if b is not None else None,
                     torch.empty((w.M, w.N), dtype=out_t, device=dev)))
    ctx = dlp.proj_create(0)
    stream = torch.cuda.Stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        e0.record(stream)
        for r in range(args.reps):
            Xd, Wd, bd, Y = sets[r % 2]
            dlp.proj_run_candidate(ctx, i, Xd, Wd, bd, w.epi, Y, stream=stream)
        e1.record(stream)
    e1.synchronize()
    dlp.proj_destroy(ctx)
    print(json.dumps({"workload": w.name, "candidate": names[i], "reps": args.reps,
                      "mean_us": round(e0.elapsed_time(e1) * 1e3 / args.reps, 3)}), flush=True)
    return 0


class WorkloadRun:
    """One workload set up for timing: P rotating buffer sets (distinct
    allocations of X, W, bias, Y; together more than twice the last-level
    cache), the plan tuned on the first call of each set, and HIP graphs
    holding R calls that cycle over the sets (plus a tail graph so that
    exactly `steps` calls are replayed)."""

    def __init__(self, ctx, w, inputs, args, dev, stream):
        import numpy as np
        import torch

        import dense_linear_projection_amd as dlp
        import synth

        X, W, b = inputs
        self.ctx, self.w, self.stream, self.args = ctx, w, stream, args
        set_bytes = w.alg_bytes()
        P = max(1, -(-(2 * LLC_BYTES) // set_bytes))      # working set > 2x the LLC
        self.P = P = min(P, 16)
        to_dev = lambda a: torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        W0 = to_dev(W)
        self.b0 = b0 = to_dev(b) if b is not None else None
        self.Xs, self.Ws, self.bs, self.Ys = [], [], [], []
        out_t = torch.float32 if w.out_dtype == synth.OUT_F32 else torch.bfloat16
        for p in range(P):
            self.Xs.append(to_dev(synth.normal_bf16((w.M, w.K), 1.0, 1000 + w.index + 100 * p)))
            self.Ws.append(W0 if p == 0 else W0.clone())
            self.bs.append(None if b0 is None else (b0 if p == 0 else b0.clone()))
            self.Ys.append(torch.empty((w.M, w.N), dtype=out_t, device=dev))
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            for p in range(P):                       # plan tuning happens on the first call
                dlp.proj_run(ctx, self.Xs[p], self.Ws[p], self.bs[p], w.epi, self.Ys[p], stream=stream)
        stream.synchronize()
        self.plan = dlp.proj_get_plan(ctx, w.M, w.N, w.K, w.epi, w.out_dtype)
        # one graph holds R calls cycling over the P buffer sets
        self.R = R = args.graph_calls or max(P, min(args.steps, 200) // P * P)
        self.idx = idx = [i % P for i in range(R)]
        self.g = self._capture(idx)
        tail = args.steps % R
        self.g_tail = self._capture([i % P for i in range(tail)]) if tail else None
        # warmup (untimed)
        for _ in range(max(1, args.warmup // R)):
            dlp.proj_graph_launch(self.g, stream=stream)
        stream.synchronize()
        torch.cuda.synchronize()

    def _capture(self, idx):
        import dense_linear_projection_amd as dlp
        return dlp.proj_graph_capture(self.ctx, [self.Xs[i] for i in idx], [self.Ws[i] for i in idx],
                                      [self.bs[i] for i in idx] if self.b0 is not None else None,
                                      [self.Ys[i] for i in idx], self.w.epi, stream=self.stream)

    def time_steps(self, steps, e0, e1) -> float:
        """Exactly `steps` calls from the graphs between HIP events recorded
        on the launch stream, with device synchronisation on both sides;
        returns milliseconds per call."""
        import torch

        import dense_linear_projection_amd as dlp
        torch.cuda.synchronize()
        e0.record(self.stream)
        for _ in range(steps // self.R):
            dlp.proj_graph_launch(self.g, stream=self.stream)
        if self.g_tail is not None:
            dlp.proj_graph_launch(self.g_tail, stream=self.stream)
        e1.record(self.stream)
        e1.synchronize()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    def close(self):
        import dense_linear_projection_amd as dlp
        dlp.proj_graph_destroy(self.g)
        if self.g_tail is not None:
            dlp.proj_graph_destroy(self.g_tail)
        self.Xs = self.Ws = self.bs = self.Ys = self.b0 = None


def roofline(w, plan, ms_per_step) -> dict:
    """The roofline object of the bench line for workload w: algorithmic
    bytes (weight-streaming workloads, M <= 64) or flops (GEMMs) per call
    over the time per call, against the published HBM or bf16 matrix peak;
    `traffic` from committed counter runs of the same kernel, if any."""
    sec = ms_per_step / 1e3
    gbs = w.alg_bytes() / sec / 1e9
    tflops = w.alg_flops() / sec / 1e12
    traffic = load_traffic(w.name, plan.split(" ")[0])
    if w.M <= 64:
        roof = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": traffic}
    else:
        roof = {"bound": "mfma", "achieved": round(tflops, 1), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(tflops / BF16_PEAK_TFLOPS, 4), "traffic": traffic}
    roof["kernel"] = plan.split(" ")[0]
    roof["avg_kernel_us"] = round(ms_per_step * 1e3, 3)
    roof["alg_bytes_per_launch"] = w.alg_bytes()
    roof["alg_flops_per_launch"] = w.alg_flops()
    return roof


def time_other_workloads(ctx, headline, args, dev, stream) -> dict:
    """The other four workloads, each set up and timed as the headline is
    (same rotation rule, graph replay and step count, same process and
    context): per workload the time per call, its roofline against its own
    bound, and the plan."""
    import torch

    import synth
    out = {}
    for w in synth.WORKLOADS:
        if w.index == headline.index:
            continue
        print("timing workload %s" % w.name, file=sys.stderr, flush=True)
        run = WorkloadRun(ctx, w, synth.workload_inputs(w), args, dev, stream)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        ms = run.time_steps(args.steps, e0, e1)
        out[w.name] = {"M": w.M, "N": w.N, "K": w.K, "epilogue": w.epi,
                       "out_dtype": "fp32" if w.out_dtype == synth.OUT_F32 else "bf16",
                       "ms_per_step": round(ms, 6), "plan": run.plan, "rotating_sets": run.P,
                       "graph_calls": run.R, "gbs": round(w.alg_bytes() / (ms / 1e3) / 1e9, 1),
                       "tflops": round(w.alg_flops() / (ms / 1e3) / 1e12, 2),
                       "roofline": roofline(w, run.plan, ms)}
        run.close()
        del run
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    return out


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", type=int, default=1, help="index into synth.WORKLOADS (0..4)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--graph-calls", type=int, default=0, help="calls per captured graph (0: auto)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain copy of known size (for counter scaling)")
    ap.add_argument("--ingest", nargs=4, metavar=("FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR", "COPY_WRITE_DIR"),
                    help="write profiles/counters_<workload>.json from rocprofv3 --pmc outputs")
    ap.add_argument("--sweep", action="store_true",
                    help="time the thirty-shape set (per load; torch alongside as context) instead of one workload")
    ap.add_argument("--sweep-steps", type=int, default=400, help="calls timed per shape in --sweep")
    ap.add_argument("--packed", type=int, default=-1, metavar="TILE16",
                    help="also time the path with W registered in the packed tile layout of 16*TILE16 rows "
                         "(packing outside the timed region; reported beside the row-major figure). "
                         "-1: the tile height of the row-major plan, for weight-streaming workloads; 0: off")
    ap.add_argument("--candidate", default="",
                    help="run the first candidate plan whose name contains this text --reps times on the "
                         "workload (for hardware counters; prints only its name and mean time)")
    ap.add_argument("--reps", type=int, default=12, help="runs for --candidate")
    ap.add_argument("--timeline", default="", metavar="TRACE_CSV",
                    help="per-call timeline of graph-replayed steps from a rocprofv3 kernel trace CSV")
    ap.add_argument("--kernels", nargs="+", default=["zero_f32_kernel", "stream_kernel", "splitk_reduce_kernel"],
                    help="for --timeline: name parts of the kernels of one call, the first one opening a call")
    ap.add_argument("--gap-us", type=float, default=20.0,
                    help="for --timeline: largest gap between replayed calls")
    ap.add_argument("--grid", nargs="*", default=[], metavar="NAME_PART:WORK_ITEMS",
                    help="for --timeline: keep only dispatches of that grid size for kernels whose name has NAME_PART")
    ap.add_argument("--near-us", type=float, default=0.0,
                    help="for --timeline: keep only calls whose kernels span within a factor of 2 of this")
    ap.add_argument("--no-workloads", action="store_true",
                    help="time only the headline workload (skip the other four)")
    ap.add_argument("--plans", nargs="+", default=[],
                    help="for --ingest: one-pass stream plans to take counters for")
    args = ap.parse_args()
    if args.timeline:
        return timeline(args)
    if args.ingest:
        return ingest_counters(args)
    if args.copy_calibration:
        return copy_calibration()
    if args.sweep:
        return sweep(args)
    if args.candidate:
        return run_candidate(args)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the projection path runs on a single GPU "
              "(sharding across GPUs is designed, not built). Run with --gpus 1.", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import dense_linear_projection_amd as dlp
    import synth

    if not os.path.exists(dlp.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()

    w = synth.WORKLOADS[args.workload]
    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    ctx = dlp.proj_create(0)
    stream = torch.cuda.Stream()

    X, W, b = synth.workload_inputs(w)
    run = WorkloadRun(ctx, w, (X, W, b), args, dev, stream)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    ms_per_step = run.time_steps(args.steps, e0, e1)   # the contract's timed region
    P, R, plan, idx = run.P, run.R, run.plan, run.idx
    Xs, Ws, bs, Ys, g, g_tail, b0 = run.Xs, run.Ws, run.bs, run.Ys, run.g, run.g_tail, run.b0
    sec = ms_per_step / 1e3

    gbs = w.alg_bytes() / sec / 1e9
    tflops = w.alg_flops() / sec / 1e12
    hbm_bound = w.M <= 64
    roof = roofline(w, plan, ms_per_step)

    # Outside the contract's timed region: the same K steps repeated TRIALS
    # times (median, min, max per step), and a warm number with one buffer
    # set, whose operands stay in the last-level cache (not an HBM rate).
    TRIALS = 5
    trial_us = []
    for _ in range(TRIALS):
        e0.record(stream)
        for _ in range(args.steps // R):
            dlp.proj_graph_launch(g, stream=stream)
        if g_tail is not None:
            dlp.proj_graph_launch(g_tail, stream=stream)
        e1.record(stream)
        e1.synchronize()
        trial_us.append(e0.elapsed_time(e1) * 1e3 / args.steps)
    trial_us.sort()
    trials = {"n": TRIALS, "median_us": round(trial_us[TRIALS // 2], 3), "min_us": round(trial_us[0], 3),
              "max_us": round(trial_us[-1], 3)}
    g_warm = dlp.proj_graph_capture(ctx, [Xs[0]] * R, [Ws[0]] * R, [bs[0]] * R if b0 is not None else None,
                                    [Ys[0]] * R, w.epi, stream=stream)
    dlp.proj_graph_launch(g_warm, stream=stream)
    reps_warm = max(1, args.steps // R)
    e0.record(stream)
    for _ in range(reps_warm):
        dlp.proj_graph_launch(g_warm, stream=stream)
    e1.record(stream)
    e1.synchronize()
    warm_s = e0.elapsed_time(e1) / 1e3 / (reps_warm * R)
    warm = {"us": round(warm_s * 1e6, 3), "gbs": round(w.alg_bytes() / warm_s / 1e9, 1),
            "tflops": round(w.alg_flops() / warm_s / 1e12, 2),
            "note": "one buffer set (P=1): operands resident in the 256 MiB last-level cache, not an HBM rate"}
    dlp.proj_graph_destroy(g_warm)

    read_floor = None
    if hbm_bound:
        read_floor = time_read_floor(ctx, Ws, idx, stream, args)
        read_floor["projection_over_floor"] = round(gbs / read_floor["gbs"], 4)

    packed = None
    if args.packed < 0 and plan.startswith("stream_"):
        args.packed = int(plan.split("_nt")[1].split("_")[0])
    if args.packed > 0:
        packed = time_packed(ctx, w, args, Xs, Ws, bs, Ys, idx, stream)

    run.close()
    del Xs, Ws, bs, Ys, g, g_tail, b0
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    others = None if args.no_workloads else time_other_workloads(ctx, w, args, dev, stream)
    dlp.proj_destroy(ctx)

    line = {
        "metric": METRIC,
        "value": round(gbs, 1) if hbm_bound else round(tflops, 2),
        "unit": "GB/s" if hbm_bound else "TFLOP/s",
        "tflops": round(tflops, 2),
        "gbs": round(gbs, 1),
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "M": w.M, "N": w.N, "K": w.K, "epilogue": w.epi,
                   "out_dtype": "fp32" if w.out_dtype == synth.OUT_F32 else "bf16",
                   "accumulate": "fp32", "rotating_sets": P, "graph_calls": R, "plan": plan},
        "roofline": roof,
        "trials": trials,
        "warm": warm,
    }
    if read_floor is not None:
        line["read_floor"] = read_floor
    if packed is not None:
        line["packed_weights"] = packed
    if others is not None:
        line["workloads"] = others
    props = torch.cuda.get_device_properties(0)
    line["device"] = {"name": props.name, "arch": getattr(props, "gcnArchName", ""),
                      "compute_units": props.multi_processor_count,
                      "peaks_used": {"hbm_gbs": HBM_PEAK_GBS, "bf16_mfma_tflops": BF16_PEAK_TFLOPS},
                      "note": "peaks are the published MI355X figures (2.4 GHz); the sustained clock under load is lower"}
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, X, W, b, args.cpu_seconds)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
