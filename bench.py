#!/usr/bin/env python3
"""Bench of the speculative-sampling verification step on one MI355X.

Workload (one "step"): one spec_verify_sample call over a full batch already resident in HBM,
B=64 requests, K=4 drafts, V=128256, bf16 logits, T=0.7 (the C3 batched-serving workload:
target N(0,3^2) + Zipf bias, draft noise std per request ~ U(0.3,2.0)). Four seeded input sets,
each held in three device copies (12 buffers, 1.77 GB), are rotated so the 256 MB Infinity Cache
cannot serve any part of a call from an earlier one (the statistics pass leaves only some rows
in it). Before the warm-up steps the bench runs the same calls for --settle-ms (default 100 ms,
untimed, reported as extra.settle_ms): the GPU takes several milliseconds of sustained load to
reach its steady clocks, and 20 warm-up steps alone left the timed ones ~10 % slower.

Prints ONE JSON line on stdout: verified draft rows/s (B*K per call), the whole call's
algorithmic HBM rate, the roofline of the dominant kernel (the streaming statistics kernel,
timed with start/stop events on its own launches inside the timed region), and the fp64 oracle
timed on this host's cores as a CPU baseline. Diagnostics go to stderr.

    python bench.py [--gpus 1] [--steps 200] [--warmup 20] [--settle-ms 100]
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from synthetic import make_contexts, make_workload  # noqa: E402

METRIC = "verified draft rows/sec and HBM GB/s (% of peak), B=64 K=4 V=128256 bf16"
HBM_PEAK_GBPS = 8000.0     # MI355X HBM3E, published
CPU_POOL_CAP = 16          # host share of one GPU


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--settle-ms", type=float, default=100.0,
                    help="untimed calls before the warm-up steps, until this much time has passed")
    ap.add_argument("--sets", type=int, default=4, help="distinct input sets")
    ap.add_argument("--copies", type=int, default=3,
                    help="device copies of each input set (all of them are rotated)")
    ap.add_argument("--cpu-repeats", type=int, default=32,
                    help="passes of the oracle over the 64 requests of set 0")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--no-secondary", action="store_true",
                    help="skip the greedy and outcome-key timings")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the C1/C2 latency, C4 throughput and C5 hit-rate figures")
    ap.add_argument("--no-c4", action="store_true",
                    help="skip C4 (its 1.32 GB input takes ~30 s to generate on the host)")
    ap.add_argument("--trace-summary", metavar="TRACE_DIR",
                    help="print the markdown summary of a rocprofv3 --kernel-trace run of this "
                         "bench and exit")
    ap.add_argument("--counter-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="print the markdown summary of two rocprofv3 --pmc runs of this bench "
                         "(FETCH_SIZE, then WRITE_SIZE) and exit")
    ap.add_argument("--issue-summary", nargs="+", metavar="PMC_DIR",
                    help="print the markdown summary of rocprofv3 --pmc runs of this bench that "
                         "collected SQ wave, wait, VALU and memory-instruction counters and "
                         "SQC_ICACHE_MISSES, and exit")
    ap.add_argument("--calib-mib", type=int, default=256,
                    help="size of one plain device-to-device copy run before timing; under "
                         "rocprofv3 --pmc its FETCH_SIZE/WRITE_SIZE calibrate the counters")
    return ap.parse_args()


# ------------------------------------------------------------------------------ counter traffic
COUNTERS_MD = os.path.join(ROOT, "profiles", "hbm_counters_all_kernels.md")
KERNEL_SOURCES = ("verify_sample.hip", "verify_greedy.hip", "predict.hip", "row_keys.hpp",
                  "spec_common.hpp", "plan.hpp")


def kernel_source_hash():
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "speculative_decoding_verification_12_amd", "csrc", f),
                  "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def counter_traffic(label):
    """Measured HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, calibrated on a plain copy) of
    the kernel launch `label` from the committed rocprofv3 counter summary, or None when that
    summary was taken on other kernel sources or does not cover it."""
    try:
        with open(COUNTERS_MD) as fh:
            for line in fh:
                f = line.split()
                if len(f) == 5 and f[0] == "traffic_bytes_per_launch" and f[1] == label and \
                        f[3] == "source_sha256_16":
                    return int(f[2]) if f[4] == kernel_source_hash() else None
    except OSError:
        return None
    return None


def _chunks(rows, V, epv, max_cv=0):
    """Chunks per row of a streaming launch (the library's plan: 256 threads, 4 vectors each,
    8 workgroups per CU on 256 CUs), to name the launches a counter run records."""
    nvec = max(V // epv, 1)
    cap = 256 * 8
    nchunk = -(-nvec // 1024)
    if rows * nchunk < 4 * cap:
        fill, finest = cap // rows, -(-nvec // 256)
        nchunk = 1 if fill < 1 else min(fill, finest)
    cv = -(-(-(-nvec // nchunk)) // 256) * 256
    if max_cv and cv > max_cv:
        cv = max_cv
    return -(-nvec // cv)


def _draw_group(B, nd):
    """Chunks per draw workgroup, as the library's plan picks them (draw_group: the fewest that
    fit every draw workgroup on the 256 CUs at 8 each, at most 4)."""
    return max(1, min(4, -(-(B * nd) // (256 * 8))))


def _draw_kernel(flags, B, nd, K=0):
    """(kernel name, workgroups) of a draw launch with template flags `flags` (keys, mixed,
    point) over B requests of nd chunks (keys add B·K workgroups on top). The one-chunk
    instance runs while its whole grid fits at 5 workgroups per CU."""
    g = _draw_group(B, nd)
    one = B * (nd + (K if flags.startswith("true") else 0)) <= 256 * 5
    name = f"sample_draw_kernel<unsigned short, {flags}, {'false' if one else 'true'}>"
    return name, B * -(-nd // g)


def bench_launches():
    """(label, kernel name prefix, workgroups, algorithmic bytes or None, workload) of every
    streaming launch the bench makes (bf16 rows)."""
    out = []
    # C1 (fp32, 4 elements a vector) and C2: one request each, statistics and draw in one launch
    for cid, K, V, epv, tname in ((1, 4, 1000, 4, "float"), (2, 5, 32000, 8, "unsigned short")):
        rows = 2 * K + 1
        out.append((f"c{cid}_sample_one_launch", f"sample_fused_kernel<{tname}>",
                    rows * _chunks(rows, V, epv) + -(-(V // epv) // 1024), rows * V * (16 // epv),
                    f"C{cid} sampling, one launch (statistics and draw)"))
    for cid, B, K, V in ((3, 64, 4, 128256), (4, 256, 8, 152064)):
        rows = B * (2 * K + 1)
        ns, nd = _chunks(rows, V, 8), -(-(V // 8) // 1024)
        ng = _chunks(B * (K + 1), V, 8, 1024)
        dname, dwg = _draw_kernel("false, false, false", B, nd)
        out += [(f"c{cid}_sample_stats", "sample_stats_kernel<unsigned short, false, false, false>",
                 rows * ns, rows * V * 2, f"C{cid} sampling, statistics pass"),
                (f"c{cid}_sample_draw", dname, dwg, None, f"C{cid} sampling, draw"),
                (f"c{cid}_greedy", "greedy_kernel<unsigned short>", B * (K + 1) * ng + B,
                 B * (K + 1) * V * 2, f"C{cid} greedy")]
        if cid == 3:
            out += [("c5_keys_stats", "sample_stats_kernel<unsigned short, true, false, false>",
                     rows * ns, rows * V * 2, "C5 verification with keys, statistics pass"),
                    ("c5_keys_draw", _draw_kernel("true, false, false", B, nd, K)[0],
                     _draw_kernel("true, false, false", B, nd, K)[1] + B * K, None,
                     "C5 verification with keys, draw and key selection"),
                    ("c3_mixed_stats", "sample_stats_kernel<unsigned short, false, true, false>",
                     rows * ns, (B // 2) * (2 * K + 1) * V * 2 + (B // 2) * (K + 1) * V * 2,
                     "C3 mixed batch (half at T = 0), statistics pass"),
                    ("c3_mixed_draw", *_draw_kernel("false, true, false", B, nd), None,
                     "C3 mixed batch, draw"),
                    ("c3_point_stats", "sample_stats_kernel<unsigned short, false, false, true>",
                     B * (K + 1) * _chunks(B * (K + 1), V, 8, 1024), None,
                     "C3 point-mass verification (lookup and full drafts), statistics pass"),
                    ("c3_point_draw", *_draw_kernel("false, false, true", B, nd), None,
                     "C3 point-mass verification, draw"),
                    ("c5_predict_stats", "predict_stats_kernel<unsigned short>",
                     B * K * _chunks(B * K, V, 8, 1024), B * K * V * 2,
                     "C5 outcome keys (and fan-out keys), statistics pass"),
                    ("c5_predict_select", "predict_select_kernel<unsigned short>", B * K, None,
                     "C5 outcome keys, selection")]
    return out


def trace_summary(trace_dir):
    """Markdown summary of a rocprofv3 --kernel-trace run of this bench: dispatches, mean and
    median duration of every streaming launch (grouped by kernel and grid), with the launch's
    algorithmic bytes over its mean duration against the 8 TB/s HBM peak."""
    import csv
    import glob
    per = {}
    for f in glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            wg = -(-int(r["Grid_Size_X"]) // max(1, int(r["Workgroup_Size_X"])))
            dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-3
            per.setdefault((r["Kernel_Name"], wg), []).append(dur)
    lines = ["| workload | kernel | workgroups | dispatches | mean us | median us | "
             "algorithmic rate |", "|---|---|---|---|---|---|---|"]
    for label, prefix, wg, alg, what in bench_launches():
        d = [v for (k, g), vs in per.items() if prefix in k and g == wg for v in vs]
        if not d:
            lines.append(f"| {what} | {prefix} | {wg} | 0 | - | - | - |")
            continue
        mean, med = float(np.mean(d)), float(np.median(d))
        rate = f"{alg / (mean * 1e-6) / 1e12:.2f} TB/s ({alg / (mean * 1e-6) / 1e9 / HBM_PEAK_GBPS:.1%})" \
            if alg else "-"
        lines.append(f"| {what} | {prefix} | {wg} | {len(d)} | {mean:.2f} | {med:.2f} | {rate} |")
    return "\n".join(lines)


def issue_summary(*dirs):
    """Markdown summary of rocprofv3 --pmc runs of this bench with the SQ wave counters
    (SQ_WAVES, SQ_WAVE_CYCLES, SQ_WAIT_ANY, SQ_WAIT_INST_ANY, SQ_ACTIVE_INST_VALU, SQ_INSTS_VALU,
    SQ_INSTS_VMEM_RD) and SQC_ICACHE_MISSES: per streaming launch, the mean wave lifetime and how
    its wave-cycles split between waiting (for memory, a barrier or a dependency), waiting to
    issue, and vector ALU work. The cycle counters count quad-cycles summed over every SIMD."""
    import csv
    import glob
    per = {}
    for d in dirs:
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            for r in csv.DictReader(open(f)):
                wg = int(r["Grid_Size"]) // max(1, int(r["Workgroup_Size"]))
                key = (r["Kernel_Name"], wg, r["Counter_Name"])
                per.setdefault(key, []).append(float(r["Counter_Value"]))

    def mean(prefix, wg, counter):
        v = [x for (k, g, c), xs in per.items() if prefix in k and g == wg and c == counter
             for x in xs]
        return (float(np.mean(v)), len(v)) if v else (None, 0)

    lines = ["| workload | kernel | workgroups | waves | cycles per wave | waiting | "
             "waiting to issue | VALU active | VALU instructions per wave | memory reads per wave "
             "| icache misses per dispatch |", "|---|---|---|---|---|---|---|---|---|---|---|"]
    for label, prefix, wg, alg, what in bench_launches():
        waves, n = mean(prefix, wg, "SQ_WAVES")
        cyc = mean(prefix, wg, "SQ_WAVE_CYCLES")[0]
        if not waves or not cyc:
            lines.append(f"| {what} | {prefix} | {wg} | - | - | - | - | - | - | - | - |")
            continue
        wait, issue, valu_c = (mean(prefix, wg, c)[0] for c in
                               ("SQ_WAIT_ANY", "SQ_WAIT_INST_ANY", "SQ_ACTIVE_INST_VALU"))
        valu_i, vmem, icm = (mean(prefix, wg, c)[0] for c in
                             ("SQ_INSTS_VALU", "SQ_INSTS_VMEM_RD", "SQC_ICACHE_MISSES"))
        share = lambda x: f"{x / cyc:.0%}" if x is not None else "-"
        perw = lambda x: f"{x / waves:.0f}" if x is not None else "-"
        icms = f"{icm:.0f}" if icm is not None else "-"
        lines.append(f"| {what} | {prefix} | {wg} | {waves:.0f} | {4 * cyc / waves:.0f} | "
                     f"{share(wait)} | {share(issue)} | {share(valu_c)} | {perw(valu_i)} | "
                     f"{perw(vmem)} | {icms} |")
    return "\n".join(lines)


def _sum_traffic(*labels):
    """Measured bytes of a call made of these launches, or None when one is not covered."""
    vals = [counter_traffic(lb) for lb in labels]
    return None if any(v is None for v in vals) else sum(vals)


def counter_summary(fetch_dir, write_dir):
    """Markdown summary of two rocprofv3 --pmc runs of this bench (FETCH_SIZE, then
    WRITE_SIZE): mean KiB per dispatch of every streaming launch, scaled by what the counters
    read for the bench's plain device-to-device copy of --calib-mib MiB, against the launch's
    algorithmic bytes; then one machine-readable line per launch for the bench's `traffic`
    fields."""
    import csv
    import glob

    def load(d, counter):
        per = {}
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            for r in csv.DictReader(open(f)):
                if r["Counter_Name"] != counter:
                    continue
                wg = int(r["Grid_Size"]) // max(1, int(r["Workgroup_Size"]))
                per.setdefault((r["Kernel_Name"], wg), []).append(float(r["Counter_Value"]))
        return per

    fetch, write = load(fetch_dir, "FETCH_SIZE"), load(write_dir, "WRITE_SIZE")
    calib_kib = 256 * 1024
    copies_f = [v for (k, wg), vs in fetch.items() if "copyBuffer" in k for v in vs]
    copies_w = [v for (k, wg), vs in write.items() if "copyBuffer" in k for v in vs]
    sf, sw = calib_kib / max(copies_f), calib_kib / max(copies_w)
    lines = [f"Calibration: the bench's plain copy of 256 MiB reads FETCH_SIZE = {max(copies_f):.1f} "
             f"KiB and WRITE_SIZE = {max(copies_w):.1f} KiB for 262144 KiB each way, so FETCH_SIZE is "
             f"scaled by {sf:.4f} and WRITE_SIZE by {sw:.4f}.", "",
             "| workload | kernel | workgroups | dispatches | read MB | write MB | algorithmic MB | "
             "measured / algorithmic |", "|---|---|---|---|---|---|---|---|"]
    machine = []
    for label, prefix, wg, alg, what in bench_launches():
        fk = [v for (k, g), vs in fetch.items() if prefix in k and g == wg for v in vs]
        wk = [v for (k, g), vs in write.items() if prefix in k and g == wg for v in vs]
        if not fk or not wk:
            lines.append(f"| {what} | {prefix} | {wg} | 0 | - | - | - | - |")
            continue
        rd = float(np.mean(fk)) * 1024 * sf
        wr = float(np.mean(wk)) * 1024 * sw
        ratio = f"{(rd + wr) / alg:.4f}" if alg else "-"
        algs = f"{alg / 1e6:.3f}" if alg else "-"
        lines.append(f"| {what} | {prefix} | {wg} | {len(fk)} | {rd / 1e6:.3f} | {wr / 1e6:.3f} | "
                     f"{algs} | {ratio} |")
        machine.append(f"traffic_bytes_per_launch {label} {int(round(rd + wr))} source_sha256_16 "
                       f"{kernel_source_hash()}")
    return "\n".join(lines + ["", "Machine-readable lines used by bench.py (dropped when the "
                               "kernel sources no longer hash to this value):", ""] + machine)


# ------------------------------------------------------------------------------ CPU baseline
_WL = None


def _oracle_requests(reqs):
    import oracle
    wl = _WL
    oracle.verify_sample(wl.target, wl.draft, wl.dtype, wl.tokens, wl.uniforms, wl.kv_len, wl.T,
                         requests=reqs)
    return len(reqs)


def cpu_baseline(wl, repeats):
    """The fp64 oracle as it is, over a fork pool on this host's cores (before any GPU use)."""
    import multiprocessing as mp
    global _WL
    _WL = wl
    workers = max(1, min(CPU_POOL_CAP, len(os.sched_getaffinity(0))))
    tasks = [b for _ in range(repeats) for b in range(wl.B)]
    slices = [tasks[i::workers] for i in range(workers)]
    ctx = mp.get_context("fork")
    with ctx.Pool(workers) as pool:
        pool.map(_oracle_requests, [[0]] * workers)          # warm the workers
        t0 = time.perf_counter()
        done = sum(pool.map(_oracle_requests, slices))
        dt = time.perf_counter() - t0
    rows = done * wl.K
    return dict(value=rows / dt, unit="verified draft rows/s", cores=workers, kind="oracle",
                sample=f"{repeats} passes over the {wl.B} requests of input set 0 "
                       f"({done} request verifications, {rows} draft rows, fp64 NumPy oracle, "
                       f"{dt:.2f} s wall on {workers} processes)")


# ------------------------------------------------------------------------------ GPU
def main():
    args = parse()
    if args.counter_summary:
        print(counter_summary(*args.counter_summary))
        return
    if args.issue_summary:
        print(issue_summary(*args.issue_summary))
        return
    if args.trace_summary:
        print(trace_summary(args.trace_summary))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the verification step runs on a single MI355X "
              "(requests are independent, so a batch splits across GPUs by request with no "
              f"exchange). --gpus {args.gpus} is not supported.", file=sys.stderr)
        sys.exit(2)

    log(f"generating {args.sets} C3 input sets")
    sets = [make_workload(3, r) for r in range(args.sets)]
    wl0 = sets[0]
    B, K, V = wl0.B, wl0.K, wl0.V
    elem = wl0.elem_bytes
    bytes_per_call = B * (2 * K + 1) * V * elem

    cpu = None
    if not args.no_cpu:
        log("oracle CPU baseline")
        cpu = cpu_baseline(wl0, args.cpu_repeats)
        log(f"cpu: {cpu['value']:.1f} rows/s on {cpu['cores']} processes")

    import torch
    import speculative_decoding_verification_12_amd as sv
    sv.load_library()
    hip = sv.hip_runtime()
    hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                        ctypes.c_void_p]
    hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log(f"device {torch.cuda.get_device_name(0)}")

    def upload(wl):
        lg = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(
            torch.bfloat16).to(dev)
        return dict(t=lg(wl.target), d=lg(wl.draft), x=torch.from_numpy(wl.tokens).to(dev),
                    u=torch.from_numpy(wl.uniforms).to(dev), kv=torch.from_numpy(wl.kv_len).to(dev))

    dsets = [upload(w) for w in sets]
    if args.calib_mib > 0:   # plain copy of known size (reads and writes calib_mib MiB once)
        src = torch.empty(args.calib_mib << 20, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    # copy-major order: buffer i holds input set i % len(sets)
    dsets = [{k: v.clone() for k, v in s.items()} if c else s
             for c in range(max(1, args.copies)) for s in dsets]
    ws = sv.new_workspace(B, K, V, 3)
    out = dict(tokens=torch.empty((B, K + 1), dtype=torch.int32, device=dev),
               tau=torch.empty(B, dtype=torch.int32, device=dev),
               kv_len=torch.empty(B, dtype=torch.int32, device=dev),
               p=torch.empty((B, K), dtype=torch.float32, device=dev),
               q=torch.empty((B, K), dtype=torch.float32, device=dev))
    T = float(wl0.T)

    def call(i, events=None):
        s = dsets[i % len(dsets)]
        sv.spec_verify_sample(s["t"], s["d"], s["x"], s["u"], s["kv"], T, ws, out=out,
                              events=events)

    # quick correctness check of what is timed (8 requests of set 0 against the oracle)
    import oracle
    call(0)
    torch.cuda.synchronize()
    ref = oracle.verify_sample(wl0.target, wl0.draft, wl0.dtype, wl0.tokens, wl0.uniforms,
                               wl0.kv_len, wl0.T, requests=range(8))
    got = out["tokens"][:8].cpu().numpy()
    for i in range(8):
        if not ref["flagged"][i] and not np.array_equal(got[i], ref["tokens"][i]):
            raise SystemExit(f"bench output differs from the oracle at request {i}")

    # events for the per-kernel timing: 4 per step
    n_ev = 4 * args.steps
    evs = (ctypes.c_void_p * n_ev)()
    ev_base = ctypes.addressof(evs)
    ev_size = ctypes.sizeof(ctypes.c_void_p)

    def ev_ptr(i):
        return ctypes.cast(ev_base + i * ev_size, ctypes.POINTER(ctypes.c_void_p))

    for i in range(n_ev):
        if hip.hipEventCreate(ev_ptr(i)) != 0:
            raise SystemExit("hipEventCreate failed")

    # settle the device's clocks under sustained load (untimed), then the W warm-up steps
    t_settle = time.perf_counter()
    n_settle = 0
    while (time.perf_counter() - t_settle) * 1e3 < args.settle_ms:
        for _ in range(64):
            call(n_settle)
            n_settle += 1
        torch.cuda.synchronize()
    settle_ms = (time.perf_counter() - t_settle) * 1e3
    for i in range(args.warmup):
        call(i)
    torch.cuda.synchronize()

    # ---- timed region: K steps, each one spec_verify_sample call, events bracketing the loop
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record()
    for i in range(args.steps):
        call(i)
    stop.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = start.elapsed_time(stop) / args.steps

    # ---- per-kernel durations: the same K steps through spec_verify_sample_ex, whose
    # kernels are launched with start/stop events (this adds launch overhead between calls, so
    # the loop's own time is not used for the headline)
    torch.cuda.synchronize()
    start.record()
    for i in range(args.steps):
        call(i, events=ev_ptr(4 * i))
    stop.record()
    torch.cuda.synchronize()
    ms_timed_entry = start.elapsed_time(stop) / args.steps

    def elapsed(a, b):
        f = ctypes.c_float()
        if hip.hipEventElapsedTime(ctypes.byref(f), evs[a], evs[b]) != 0:
            raise SystemExit("hipEventElapsedTime failed")
        return f.value

    stats_ms = np.array([elapsed(4 * i, 4 * i + 1) for i in range(args.steps)])
    draw_ms = np.array([elapsed(4 * i + 2, 4 * i + 3) for i in range(args.steps)])

    # hot: one input set only (Infinity Cache may serve part of it)
    start.record()
    for i in range(args.steps):
        call(0)
    stop.record()
    torch.cuda.synchronize()
    ms_hot = start.elapsed_time(stop) / args.steps

    stats_avg_s = float(stats_ms.mean()) * 1e-3
    achieved = bytes_per_call / stats_avg_s / 1e9
    rows_per_s = B * K / (ms_per_step * 1e-3)
    call_gbps = bytes_per_call / (ms_per_step * 1e-3) / 1e9

    extra = dict(settle_ms=round(settle_ms, 1), settle_calls=n_settle,
                 ms_per_step_timed_entry=round(ms_timed_entry, 5),
                 ms_per_step_hot_one_set=round(ms_hot, 5),
                 wall_ms_per_step=round(wall / args.steps * 1e3, 5),
                 stats_kernel_us=dict(mean=round(float(stats_ms.mean()) * 1e3, 3),
                                      median=round(float(np.median(stats_ms)) * 1e3, 3),
                                      p90=round(float(np.percentile(stats_ms, 90)) * 1e3, 3)),
                 draw_kernel_us=dict(mean=round(float(draw_ms.mean()) * 1e3, 3),
                                     median=round(float(np.median(draw_ms)) * 1e3, 3)),
                 bytes_per_call=bytes_per_call,
                 call_hbm_gbps=round(call_gbps, 1),
                 call_pct_of_peak=round(100 * call_gbps / HBM_PEAK_GBPS, 2),
                 draw_kernel_traffic=counter_traffic("c3_sample_draw"))

    if not args.no_secondary:
        extra.update(secondary(sv, torch, dev, hip, sets, dsets, ws, args))
    if not args.no_configs:
        extra.update(other_configs(sv, torch, dev, args))

    for i in range(n_ev):
        hip.hipEventDestroy(evs[i])

    line = {
        "metric": METRIC,
        "value": round(rows_per_s, 1),
        "unit": "verified draft rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "C3 batched serving: spec_verify_sample, B=64 K=4 V=128256 bf16 "
                               f"T=0.7, {len(dsets)} rotated buffers ({len(sets)} input sets)",
                   "B": B, "K": K, "V": V, "temperature": T, "input_sets": len(sets),
                   "rotated_buffers": len(dsets)},
        "hbm_gbps": round(call_gbps, 1),
        "pct_of_hbm_peak": round(100 * call_gbps / HBM_PEAK_GBPS, 2),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": counter_traffic("c3_sample_stats"),
                     "kernel": "sample_stats_kernel<bf16>",
                     "bytes_per_launch": bytes_per_call,
                     "avg_launch_us": round(stats_avg_s * 1e6, 3),
                     "call_frac": round(call_gbps / HBM_PEAK_GBPS, 4)},
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(line), flush=True)


def other_configs(sv, torch, dev, args):
    """The other workloads' own figures: C1 and C2 per-call latency (one request each; device
    time between events around every call, and host wall time of a launch-and-wait), C4
    throughput with its share of bonus-path requests, and the C5 outcome-key hit rates."""
    res = {}
    steps = max(50, args.steps)

    def upload(w):
        if w.dtype == "bf16":
            lg = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(
                torch.bfloat16).to(dev)
        else:
            lg = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
        return dict(t=lg(w.target), d=lg(w.draft), x=torch.from_numpy(w.tokens).to(dev),
                    u=torch.from_numpy(w.uniforms).to(dev),
                    kv=torch.from_numpy(w.kv_len).to(dev))

    def outputs(B, K):
        return dict(tokens=torch.empty((B, K + 1), dtype=torch.int32, device=dev),
                    tau=torch.empty(B, dtype=torch.int32, device=dev),
                    kv_len=torch.empty(B, dtype=torch.int32, device=dev),
                    p=torch.empty((B, K), dtype=torch.float32, device=dev),
                    q=torch.empty((B, K), dtype=torch.float32, device=dev))

    def latency(fn, n_sets):
        """Per call: device us between events around it, and host wall us of launch + wait."""
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(steps)]
        for i in range(20):
            fn(i % n_sets)
        torch.cuda.synchronize()
        wall = []
        for i in range(steps):
            t0 = time.perf_counter()
            ev[i][0].record()
            fn(i % n_sets)
            ev[i][1].record()
            ev[i][1].synchronize()
            wall.append((time.perf_counter() - t0) * 1e6)
        dev_us = np.array([a.elapsed_time(b) * 1e3 for a, b in ev])
        wall = np.array(wall)
        return dict(device_us_median=round(float(np.median(dev_us)), 2),
                    device_us_p90=round(float(np.percentile(dev_us, 90)), 2),
                    wall_us_median=round(float(np.median(wall)), 2),
                    wall_us_p90=round(float(np.percentile(wall, 90)), 2))

    # ---- C1 (fp32, V=1000) and C2 (bf16, V=32000): one request per call
    for cid, name in ((1, "c1_tiny"), (2, "c2_latency")):
        log(f"C{cid} per-call latency")
        n_sets = 64
        wls = [make_workload(cid, r) for r in range(n_sets)]
        ds = [upload(w) for w in wls]
        B, K, V = wls[0].B, wls[0].K, wls[0].V
        ws = sv.new_workspace(B, K, V)
        out = outputs(B, K)
        T = float(wls[0].T)

        # calls through the C ABI with arguments marshalled once per input set (the binding's
        # per-call argument checks alone cost several microseconds of host time, which the
        # device then spends idle between the events)
        samp_calls = [sv.prepared_sample(s["t"], s["d"], s["x"], s["u"], s["kv"], T, ws, out)
                      for s in ds]
        greedy_calls = [sv.prepared_greedy(s["t"], s["x"], s["kv"], ws, out) for s in ds]

        def samp_binding(i):
            s = ds[i]
            sv.spec_verify_sample(s["t"], s["d"], s["x"], s["u"], s["kv"], T, ws, out=out)

        res[name] = dict(B=B, K=K, V=V, dtype=wls[0].dtype, T=T,
                         sample_warm=latency(lambda i: samp_calls[i](), 1),
                         sample_rotated=latency(lambda i: samp_calls[i](), n_sets),
                         greedy_warm=latency(lambda i: greedy_calls[i](), 1),
                         greedy_rotated=latency(lambda i: greedy_calls[i](), n_sets),
                         sample_rotated_via_binding_checks=latency(samp_binding, n_sets),
                         rotated_sets=n_sets)
        # the same sampling call captured once into a HIP graph and replayed (the caller's way
        # of removing host launch cost from a latency-bound loop; the library records no
        # memset node, so replays are exact)
        static = {k: v.clone() for k, v in ds[0].items()}

        def samp_static():
            sv.spec_verify_sample(static["t"], static["d"], static["x"], static["u"],
                                  static["kv"], T, ws, out=out)

        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            samp_static()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            samp_static()
        torch.cuda.synchronize()
        res[name]["sample_graph_replay"] = latency(lambda i: graph.replay(), 1)
        del graph

    # ---- C4: B=256, K=8, V=152064 bf16, T=1; even requests accept every draft (bonus path).
    # One input set of 1.32 GB, five times the Infinity Cache, so calls cannot hit it.
    if not args.no_c4:
        log("C4 large batch (generating 1.32 GB of logits on the host)")
        w4 = make_workload(4, 0)
        d4 = upload(w4)
        B, K, V = w4.B, w4.K, w4.V
        ws = sv.new_workspace(B, K, V)
        out = outputs(B, K)
        T = float(w4.T)
        start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        n4 = max(20, args.steps // 4)
        for fn_name in ("sample", "greedy"):
            def fn():
                if fn_name == "sample":
                    sv.spec_verify_sample(d4["t"], d4["d"], d4["x"], d4["u"], d4["kv"], T, ws,
                                          out=out)
                else:
                    sv.spec_verify_greedy(d4["t"], d4["x"], d4["kv"], ws, out=out)
            # the host generation above left the GPU idle: settle its clocks first (untimed)
            t_settle = time.perf_counter()
            while (time.perf_counter() - t_settle) * 1e3 < args.settle_ms / 2:
                for _ in range(8):
                    fn()
                torch.cuda.synchronize()
            start.record()
            for _ in range(n4):
                fn()
            stop.record()
            torch.cuda.synchronize()
            ms = start.elapsed_time(stop) / n4
            nbytes = B * ((2 * K + 1) if fn_name == "sample" else (K + 1)) * V * 2
            tau = out["tau"].cpu().numpy()
            res.setdefault("c4_large", dict(B=B, K=K, V=V, T=T))[fn_name] = dict(
                ms_per_call=round(ms, 5), rows_per_s=round(B * K / (ms * 1e-3), 1),
                bytes_per_call=nbytes, hbm_gbps=round(nbytes / (ms * 1e-3) / 1e9, 1),
                frac_of_hbm_peak=round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                bonus_path_share=round(float(np.mean(tau == K + 1)), 4),
                mean_tau=round(float(tau.mean()), 3),
                traffic=(_sum_traffic("c4_sample_stats", "c4_sample_draw")
                         if fn_name == "sample" else counter_traffic("c4_greedy")))
        del d4

    # ---- C5 hit rates: keys (F=3, every slot, draft token kept) against the outcome of the
    # verification of the same round; a round is a hit when a draft was rejected (a < K) and
    # the placed token is one of slot a's keys (all-kept rounds have no key: misses)
    log("C5 outcome-key hit rates")
    F = 3
    for mode, Tm in (("sample", 1.0), ("greedy", 0.0)):
        hits = rej = tot = 0
        for r in range(4):
            w5 = make_workload(5, r, mode)
            d5 = upload(w5)
            B, K, V = w5.B, w5.K, w5.V
            ws = sv.new_workspace(B, K, V, F)
            out = outputs(B, K)
            if mode == "sample":
                sv.spec_verify_sample(d5["t"], d5["d"], d5["x"], d5["u"], d5["kv"], Tm, ws,
                                      out=out)
            else:
                sv.spec_verify_greedy(d5["t"], d5["x"], d5["kv"], ws, out=out)
            keys = sv.spec_predict_outcomes(d5["d"], F, Tm, ws)["keys"]
            torch.cuda.synchronize()
            tau = out["tau"].cpu().numpy()
            tok = out["tokens"].cpu().numpy()
            kk = keys.cpu().numpy()
            for b in range(B):
                a = int(tau[b]) - 1
                tot += 1
                if a < K:
                    rej += 1
                    hits += int(tok[b, a] in kk[b, a])
        res[f"c5_hit_rate_T{Tm:g}"] = dict(rounds=4, requests=tot, hit_rate=round(hits / tot, 4),
                                           hit_rate_rejected_rounds=round(hits / max(rej, 1), 4),
                                           F=F, draft_token_skipped=False)
    return res


def secondary(sv, torch, dev, hip, sets, dsets, ws, args):
    """Greedy verification on C3 and outcome keys on C5 (F=3), events around each call."""
    res = {}
    wl0 = sets[0]
    B, K, V = wl0.B, wl0.K, wl0.V
    steps = max(20, args.steps // 2)
    xg = [torch.from_numpy(make_workload(3, r, "greedy").tokens).to(dev) for r in range(len(sets))]
    outg = dict(tokens=torch.empty((B, K + 1), dtype=torch.int32, device=dev),
                tau=torch.empty(B, dtype=torch.int32, device=dev),
                kv_len=torch.empty(B, dtype=torch.int32, device=dev))
    for i in range(10):
        s = dsets[i % len(dsets)]
        sv.spec_verify_greedy(s["t"], xg[i % len(xg)], s["kv"], ws, out=outg)
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for i in range(steps):
        s = dsets[i % len(dsets)]
        sv.spec_verify_greedy(s["t"], xg[i % len(xg)], s["kv"], ws, out=outg)
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / steps
    gb = B * (K + 1) * V * 2
    res["greedy_c3"] = dict(ms_per_call=round(ms, 5), rows_per_s=round(B * K / (ms * 1e-3), 1),
                            hbm_gbps=round(gb / (ms * 1e-3) / 1e9, 1), bytes_per_call=gb,
                            traffic=counter_traffic("c3_greedy"))

    log("C5 outcome keys")
    c5 = [make_workload(5, r) for r in range(8)]
    d5 = [torch.from_numpy(np.ascontiguousarray(w.draft).view(np.int16)).view(
        torch.bfloat16).to(dev) for w in c5]
    F = 3
    outp = dict(keys=torch.empty((B, K, F), dtype=torch.int32, device=dev),
                key_prob=torch.empty((B, K, F), dtype=torch.float32, device=dev))
    # generating the inputs left the GPU idle: settle its clocks first (untimed)
    t_settle, n = time.perf_counter(), 0
    while (time.perf_counter() - t_settle) * 1e3 < args.settle_ms / 2:
        for _ in range(32):
            sv.spec_predict_outcomes(d5[n % 8], F, 1.0, ws, out=outp)
            n += 1
        torch.cuda.synchronize()
    for Tp in (1.0, 0.0):
        for i in range(10):
            sv.spec_predict_outcomes(d5[i % 8], F, Tp, ws, out=outp)
        torch.cuda.synchronize()
        start.record()
        for i in range(steps):
            sv.spec_predict_outcomes(d5[i % 8], F, Tp, ws, out=outp)
        stop.record()
        torch.cuda.synchronize()
        ms = start.elapsed_time(stop) / steps
        pb = B * K * V * 2
        res[f"predict_c5_T{Tp:g}"] = dict(ms_per_call=round(ms, 5),
                                           keys_per_s=round(B * K * F / (ms * 1e-3), 1),
                                           hbm_gbps=round(pb / (ms * 1e-3) / 1e9, 1),
                                           bytes_per_call=pb,
                                           traffic=_sum_traffic("c5_predict_stats",
                                                                "c5_predict_select"))

    # per-slot fan-out with the draft token skipped (two candidates per slot, the D3D page's
    # setting), then the lookup of each outcome's prepared continuation
    log("C5 fan-out keys and outcome lookup")
    x5 = [torch.from_numpy(w.tokens).to(dev) for w in c5]
    fan = [2] * K
    S = sum(fan)
    outf = dict(keys=torch.empty((B, S), dtype=torch.int32, device=dev),
                key_prob=torch.empty((B, S), dtype=torch.float32, device=dev))
    for i in range(10):
        sv.spec_predict_fanout(d5[i % 8], fan, 1.0, ws, draft_tokens=x5[i % 8], out=outf)
    torch.cuda.synchronize()
    start.record()
    for i in range(steps):
        sv.spec_predict_fanout(d5[i % 8], fan, 1.0, ws, draft_tokens=x5[i % 8], out=outf)
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / steps
    pb = B * K * V * 2
    res["fanout_c5_T1"] = dict(fanout=fan, draft_token_skipped=True, ms_per_call=round(ms, 5),
                               keys_per_s=round(B * S / (ms * 1e-3), 1),
                               hbm_gbps=round(pb / (ms * 1e-3) / 1e9, 1), bytes_per_call=pb)
    slot = torch.empty(B, dtype=torch.int32, device=dev)
    for i in range(10):
        sv.spec_outcome_lookup(outg["tau"], outg["tokens"], outf["keys"], fan, True, out=slot)
    torch.cuda.synchronize()
    start.record()
    for i in range(steps):
        sv.spec_outcome_lookup(outg["tau"], outg["tokens"], outf["keys"], fan, True, out=slot)
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / steps
    res["outcome_lookup"] = dict(ms_per_call=round(ms, 5),
                                 outcomes_per_s=round(B / (ms * 1e-3), 1))

    # C5: verification plus keys (F=3, draft token skipped) from the same pass over the draft
    # rows, against the two separate calls on the same inputs
    log("C5 verification with keys from the same pass")
    lg = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(
        torch.bfloat16).to(dev)
    full5 = [dict(t=lg(w.target), d=d5[r], x=x5[r], u=torch.from_numpy(w.uniforms).to(dev),
                  kv=torch.from_numpy(w.kv_len).to(dev)) for r, w in enumerate(c5[:4])]
    out = dict(tokens=torch.empty((B, K + 1), dtype=torch.int32, device=dev),
               tau=torch.empty(B, dtype=torch.int32, device=dev),
               kv_len=torch.empty(B, dtype=torch.int32, device=dev),
               p=torch.empty((B, K), dtype=torch.float32, device=dev),
               q=torch.empty((B, K), dtype=torch.float32, device=dev))
    outk = dict(out, keys=torch.empty((B, K, F), dtype=torch.int32, device=dev),
                key_prob=torch.empty((B, K, F), dtype=torch.float32, device=dev))
    T5 = float(c5[0].T)

    def fused(i):
        s = full5[i % 4]
        sv.spec_verify_sample_keys(s["t"], s["d"], s["x"], s["u"], s["kv"], T5, F, ws,
                                   exclude_draft=True, out=outk)

    def separate(i):
        s = full5[i % 4]
        sv.spec_verify_sample(s["t"], s["d"], s["x"], s["u"], s["kv"], T5, ws, out=out)
        sv.spec_predict_outcomes(s["d"], F, T5, ws, out=outp)

    for name, fn in (("fused", fused), ("separate", separate)):
        for i in range(10):
            fn(i)
        torch.cuda.synchronize()
        start.record()
        for i in range(steps):
            fn(i)
        stop.record()
        torch.cuda.synchronize()
        res.setdefault("sample_keys_c5", {})[f"{name}_ms_per_call"] = round(
            start.elapsed_time(stop) / steps, 5)
    # C3 as a mixed batch: half the requests at T = 0 (their draft rows are not read)
    log("C3 mixed batch, half greedy")
    temps = torch.tensor([0.0 if b % 2 == 0 else float(wl0.T) for b in range(B)],
                         dtype=torch.float32, device=dev)
    outm = dict(tokens=torch.empty((B, K + 1), dtype=torch.int32, device=dev),
                tau=torch.empty(B, dtype=torch.int32, device=dev),
                kv_len=torch.empty(B, dtype=torch.int32, device=dev),
                p=torch.empty((B, K), dtype=torch.float32, device=dev),
                q=torch.empty((B, K), dtype=torch.float32, device=dev))
    for i in range(10):
        s = dsets[i % len(dsets)]
        sv.spec_verify_mixed(s["t"], s["d"], s["x"], s["u"], s["kv"], temps, ws, out=outm)
    torch.cuda.synchronize()
    start.record()
    for i in range(steps):
        s = dsets[i % len(dsets)]
        sv.spec_verify_mixed(s["t"], s["d"], s["x"], s["u"], s["kv"], temps, ws, out=outm)
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / steps
    mb_bytes = (B // 2) * (2 * K + 1) * V * 2 + (B - B // 2) * (K + 1) * V * 2
    res["mixed_c3_half_greedy"] = dict(ms_per_call=round(ms, 5),
                                       rows_per_s=round(B * K / (ms * 1e-3), 1),
                                       bytes_per_call=mb_bytes,
                                       hbm_gbps=round(mb_bytes / (ms * 1e-3) / 1e9, 1),
                                       traffic=_sum_traffic("c3_mixed_stats", "c3_mixed_draw"))

    # paged KV-cache rewind of both caches after a C3 round (block size 16)
    log("KV-cache rewind")
    bs = 16
    mb = (4096 + K + 1) // bs + 1
    tab0 = torch.arange(B * mb, dtype=torch.int32, device=dev).reshape(B, mb)
    tab = tab0.clone()
    alloc = (dsets[0]["kv"] + K + 1).to(torch.int32)
    kvo = torch.empty(B, dtype=torch.int32, device=dev)
    kvo.copy_(dsets[0]["kv"] + 2)
    rw = dict(freed=torch.empty(B * mb, dtype=torch.int32, device=dev),
              offsets=torch.empty(B + 1, dtype=torch.int32, device=dev))
    for i in range(10):
        sv.spec_kv_rewind(tab, bs, alloc, kvo, out=rw)
    torch.cuda.synchronize()
    start.record()
    for i in range(steps):
        sv.spec_kv_rewind(tab, bs, alloc, kvo, out=rw)
    stop.record()
    torch.cuda.synchronize()
    res["kv_rewind_c3"] = dict(block_size=bs, ms_per_call=round(start.elapsed_time(stop) / steps, 5))

    # a round without a draft model: prompt-lookup drafts from 64 histories of 1k-16k tokens
    # (prompt, then output quoting earlier spans), then verification of those drafts against the
    # C3 target rows at C3's temperature and at T = 0
    log("prompt-lookup drafts and point-mass verification")
    ctx_np, lens_np = make_contexts(4242, B, 16384, 1024, 16384, V)
    ctx, lens = torch.from_numpy(ctx_np).to(dev), torch.from_numpy(lens_np).to(dev)
    outd = dict(tokens=torch.empty((B, K), dtype=torch.int32, device=dev),
                len=torch.empty(B, dtype=torch.int32, device=dev),
                ngram=torch.empty(B, dtype=torch.int32, device=dev),
                src=torch.empty(B, dtype=torch.int32, device=dev))

    def timed(fn):
        for i in range(10):
            fn(i)
        torch.cuda.synchronize()
        start.record()
        for i in range(steps):
            fn(i)
        stop.record()
        torch.cuda.synchronize()
        return start.elapsed_time(stop) / steps

    ms = timed(lambda i: sv.spec_ngram_draft(ctx, lens, 4, 1, K, out=outd))
    dl = outd["len"].cpu().numpy()
    res["ngram_draft_64x16k"] = dict(ms_per_call=round(ms, 5), n_max=4, n_min=1, K=K,
                                     context_tokens=int(lens_np.sum()),
                                     matched=int((dl > 0).sum()),
                                     mean_draft_len=round(float(dl.mean()), 3))
    outp = dict(tokens=torch.empty((B, K + 1), dtype=torch.int32, device=dev),
                tau=torch.empty(B, dtype=torch.int32, device=dev),
                kv_len=torch.empty(B, dtype=torch.int32, device=dev),
                p=torch.empty((B, K), dtype=torch.float32, device=dev),
                q=torch.empty((B, K), dtype=torch.float32, device=dev))
    pb = int(((dl + 1) * V * 2).sum())
    rp = dict(bytes_per_call=pb, mean_draft_len=round(float(dl.mean()), 3))
    for name, T in (("T", float(wl0.T)), ("T0", 0.0)):
        ms = timed(lambda i: sv.spec_verify_point(dsets[i % len(dsets)]["t"], outd["tokens"],
                                                  outd["len"], dsets[i % len(dsets)]["u"],
                                                  dsets[i % len(dsets)]["kv"], T, ws, out=outp))
        rp[f"{name}_ms_per_call"] = round(ms, 5)
        rp[f"{name}_hbm_gbps"] = round(pb / (ms * 1e-3) / 1e9, 1)
    ms = timed(lambda i: (sv.spec_ngram_draft(ctx, lens, 4, 1, K, out=outd),
                          sv.spec_verify_point(dsets[i % len(dsets)]["t"], outd["tokens"],
                                               outd["len"], dsets[i % len(dsets)]["u"],
                                               dsets[i % len(dsets)]["kv"], float(wl0.T), ws,
                                               out=outp)))
    rp["round_T_ms_per_call"] = round(ms, 5)
    res["point_verify_c3_lookup_drafts"] = rp
    # every slot drafted: the same bytes as greedy, against the C3 sampling call's (2K+1) rows
    fb = B * (K + 1) * V * 2
    ms = timed(lambda i: sv.spec_verify_point(dsets[i % len(dsets)]["t"], dsets[i % len(dsets)]["x"],
                                              None, dsets[i % len(dsets)]["u"],
                                              dsets[i % len(dsets)]["kv"], float(wl0.T), ws,
                                              out=outp))
    res["point_verify_c3_full_K"] = dict(ms_per_call=round(ms, 5), bytes_per_call=fb,
                                         rows_per_s=round(B * K / (ms * 1e-3), 1),
                                         hbm_gbps=round(fb / (ms * 1e-3) / 1e9, 1))
    # the counter run records the lookup-draft and full-draft calls of this grid together
    res["point_verify_c3_traffic_mean_of_both"] = _sum_traffic("c3_point_stats", "c3_point_draw")

    vb = B * (2 * K + 1) * V * 2
    r5 = res["sample_keys_c5"]
    r5.update(F=F, draft_token_skipped=True, bytes_per_call=vb,
              hbm_gbps=round(vb / (r5["fused_ms_per_call"] * 1e-3) / 1e9, 1),
              rows_per_s=round(B * K / (r5["fused_ms_per_call"] * 1e-3), 1),
              traffic=_sum_traffic("c5_keys_stats", "c5_keys_draw"))
    # every line that streams logits also states its algorithmic rate as a fraction of the
    # 8 TB/s HBM peak; the prompt-lookup drafter reads a few MB and is bound by latency instead
    for entry in res.values():
        if not isinstance(entry, dict):
            continue
        for key in [k for k in entry if k.endswith("hbm_gbps")]:
            entry[key[:-len("hbm_gbps")] + "frac_of_hbm_peak"] = round(entry[key] / HBM_PEAK_GBPS, 4)
    res["ngram_draft_64x16k"]["bound"] = "latency"
    return res


if __name__ == "__main__":
    main()
