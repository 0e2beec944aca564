"""Benchmark: MoE expert-parallel shuffle (route plan + dispatch + combine) on one MI355X.

One step = one pass of the whole path over one batch: moe_route_plan (histogram,
scan, segment descriptors), moe_dispatch (single hop, or the two hops of node
deduplication on the DeepSeek-V3-like workload) and moe_combine (bf16 out),
with the identity expert between dispatch and combine.  Inputs are resident in
HBM before any timing starts.

Default workload: the DeepSeek-V3-like multi-node shuffle (T=16384, H=7168,
E=256, k=8, R=64 in 8 virtual nodes, node deduplication), the largest
configuration; the OLMoE-like, Qwen3-like and non-divisible workloads are
measured the same way in the same run (`per_config`).

Timing protocol (`value`):
  * W warmup steps, then EXACTLY K timed steps, bracketed by synchronize.
  * Before each timed phase the last-level cache (256 MB MALL) is flushed:
    a 1 GiB scratch buffer is written, then a second 1 GiB buffer is read, so
    the phase finds neither its inputs nor dirty flush lines in the cache.
    The flush is not timed.
  * Phase 1 is route plan + dispatch, phase 2 the combine, each between two
    hipEventRecord markers on the step's stream.  A marker interval also
    holds the launch latency of the phase's first kernel (a few us), which
    back-to-back kernels hide; it is not subtracted.
  * value = algorithmic bytes per step / (median phase-1 time + median
    phase-2 time); ms_per_step is that sum.  Mean, p10 and p90 are given for
    each phase.

Other figures in the same line:
  kernels      every kernel's launches in K more flushed steps, each launch
               timed by the library with HIP events bound to the kernel's own
               start and end (moe_plan_timing): launches per step, mean
               duration, algorithmic bytes, GB/s and fraction of 8 TB/s.
               (Bound events add a few us of gap after each launch, so that
               pass gives kernel durations, not phase times.)
  roofline     the kernel with the most time per step (of those that move the
               payload): its algorithmic bytes per launch / its mean launch
               duration.  traffic = its HBM bytes per launch from the
               rocprofv3 FETCH_SIZE / WRITE_SIZE summary under profiles/,
               scaled by the copy calibration; null once the kernel sources
               have changed since the counters were taken.
  schedules    back-to-back steps without flushes, over buffer sets cycled so
               that the sets' inputs total at least 4x the MALL: serial (one
               stream), two_in_flight (step i on stream i mod 2), staggered
               (as two_in_flight, each dispatch after the previous step's
               dispatch) and plan_ahead (each route plan on a second stream
               during the previous step's movement).
  copy_ceiling a plain device-to-device copy (torch copy_) of the step's
               bytes, half read and half written, over buffer pairs cycled
               past the MALL.
  cpu_baseline the oracle (numpy, as it stands) on this host's cores, on the
               headline workload: whole passes until --cpu-seconds is spent.

Algorithmic bytes (payload rows only):
  dispatch single hop  (T + T*k) * 2H
  dispatch with dedup  (T + 2D + T*k) * 2H   (D staging rows, from the plan)
  combine              (T*k + T) * 2H

Helper modes (no GPU needed): --summarize-trace and --summarize-pmc turn
rocprofv3 CSV output into the short summaries kept under profiles/.
"""

from __future__ import annotations

import argparse
import csv
import dataclasses
import hashlib
import json
import math
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MALL_BYTES = 256 << 20   # MI355X last-level cache (AMD Infinity Cache)
FLUSH_BYTES = 1 << 30
MAX_SETS = 256
METRIC = "dispatch+combine effective GB/s and % of HBM peak, 1 MI355X"
SCHEDULES = ("serial", "two_in_flight", "staggered", "plan_ahead")
PROFILES = os.path.join(ROOT, "profiles")
# Each kernel is compiled in one translation unit (its .hip file plus the
# headers every unit includes); a traffic summary is current for a kernel
# while that unit's sources are unchanged.
KERNEL_HEADERS = ("combine_shuffling_amd/csrc/move_body.h", "combine_shuffling_amd/csrc/plan_body.h",
                  "combine_shuffling_amd/csrc/moe_device.h",
                  "combine_shuffling_amd/csrc/moe_internal.h", "include/moe_shuffle.h")
KERNEL_UNITS = ("move.hip", "pipeline.hip", "route_plan.hip")
# Kernels that carry no payload rows (plan metadata, counters).
PLAN_KERNELS = ("route_count_kernel", "route_scan_kernel", "route_assign_kernel",
                "traffic_clear_kernel", "traffic_kernel", "counters_clear_kernel")


def parse(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="dsv3",
                    help="tiny | olmoe | qwen3 | dsv3 | nondiv (default: dsv3, the DeepSeek-V3-like "
                         "multi-node shuffle with node deduplication)")
    ap.add_argument("--configs", default="olmoe,qwen3,nondiv",
                    help="further workloads measured the same way in this run, comma separated, "
                         "or 'none'")
    ap.add_argument("--payload", choices=("bf16", "fp8"), default="bf16",
                    help="row payload: bf16, or fp8 (OCP E4M3 codes + one float32 scale per "
                         "128-element block; with node dedup, the staging rows are fp8 too)")
    ap.add_argument("--load-aware-forwarders", action="store_true",
                    help="node-deduplicated workloads: choose forwarders by load")
    ap.add_argument("--hier-combine", action="store_true",
                    help="node-deduplicated workloads: two-hop combine (fp32 partial per staging "
                         "row, then the sum over the token's nodes)")
    ap.add_argument("--pipeline", action="store_true",
                    help="single-hop workloads: route, dispatch and combine of every band of "
                         "tokens in one persistent launch (banded plan)")
    ap.add_argument("--band-tokens", type=int, default=2048,
                    help="tokens per band with --pipeline (a multiple of 256)")
    ap.add_argument("--single-hop", action="store_true",
                    help="plan a workload with virtual nodes (dsv3) as one node: the same routing "
                         "moved by the single-hop gather, the lower bound on its bytes")
    ap.add_argument("--no-schedules", action="store_true",
                    help="leave out the passes that do not flush before each phase (the back-to-back "
                         "schedules, the copy ceiling and olmoe's MALL-resident combine), so that in "
                         "a profiler run every traced launch runs in the flushed protocol")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--sets", type=int, default=0, help="buffer sets cycled by the schedules (0: auto)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain elementwise copy of MIB MiB (read MIB, write MIB) a few "
                         "times, to scale hardware byte counters against a known size")
    ap.add_argument("--summarize-trace", nargs=2, metavar=("KERNEL_STATS_CSV", "OUT"),
                    help="write a kernel-duration summary of a rocprofv3 --stats CSV")
    ap.add_argument("--summarize-pmc", nargs=5,
                    metavar=("FETCH_CSV", "WRITE_CSV", "COPY_FETCH_CSV", "COPY_WRITE_CSV", "OUT"),
                    help="write the per-launch HBM traffic summary of two rocprofv3 --pmc runs "
                         "(FETCH_SIZE, WRITE_SIZE) scaled by the copy calibration runs")
    ap.add_argument("--copy-mib", type=int, default=1024,
                    help="size the copy calibration ran with (--copy-calibration MIB)")
    ap.add_argument("--command", default="", help="command line recorded in a summary")
    return ap.parse_args(argv)


_KERNEL_DEF = re.compile(r"__global__\s+(?:__launch_bounds__\([^)]*\)\s+)?void\s+(\w+)\s*\(")


def unit_kernels():
    """Kernel names of each translation unit: those its .hip file defines, and
    those a shared header defines that the file names (launches)."""
    def read(rel):
        with open(os.path.join(ROOT, rel)) as f:
            return f.read()

    in_headers = set()
    for rel in KERNEL_HEADERS:
        in_headers |= set(_KERNEL_DEF.findall(read(rel)))
    units = {}
    for unit in KERNEL_UNITS:
        src = read("combine_shuffling_amd/csrc/" + unit)
        units[unit] = set(_KERNEL_DEF.findall(src)) | {
            k for k in in_headers if re.search(r"\b%s\b" % k, src)}
    return units


def kernel_unit(kernel):
    """The .hip file whose translation unit holds `kernel` (short or full name)."""
    short = _short(kernel).split("<")[0]
    hits = [u for u, names in unit_kernels().items() if short in names]
    if len(hits) != 1:
        raise ValueError(f"kernel {short!r} found in {len(hits)} translation units")
    return hits[0]


def kernel_source_hash(unit):
    """Hash of the sources one translation unit is compiled from."""
    h = hashlib.sha256()
    for rel in ("combine_shuffling_amd/csrc/" + unit,) + KERNEL_HEADERS:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def copy_calibration(mib):
    """torch.mul(a, 1, out=b) over MIB MiB of bf16: a plain copy kernel of known size."""
    import torch

    dev = torch.device("cuda:0")
    n = mib * (1 << 20) // 2
    a = torch.randn(n, device=dev).to(torch.bfloat16)
    b = torch.empty_like(a)
    for _ in range(5):
        torch.mul(a, 1.0, out=b)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration": {"kernel": "torch elementwise mul (bf16)",
                                           "read_bytes": n * 2, "write_bytes": n * 2,
                                           "launches": 5}}), flush=True)


def copy_ceiling(torch, dev, half_bytes, steps):
    """Wall time of a plain device-to-device copy of half_bytes (torch copy_),
    over pairs of buffers cycled so the sources total at least 4x the MALL."""
    n = half_bytes // 2
    pairs = max(2, math.ceil(4 * MALL_BYTES / half_bytes))
    src = [torch.empty(n, dtype=torch.int16, device=dev).fill_(i) for i in range(pairs)]
    dst = [torch.empty_like(a) for a in src]
    for i in range(2 * pairs):
        dst[i % pairs].copy_(src[i % pairs])
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        dst[i % pairs].copy_(src[i % pairs])
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    del src, dst
    torch.cuda.empty_cache()
    return {"kernel": "torch copy_ (device to device)", "bytes": 2 * half_bytes,
            "buffer_pairs": pairs, "ms": round(ms, 5),
            "GB/s": round(2 * half_bytes / (ms * 1e-3) / 1e9, 1)}


def _pmc_means(path, counter):
    """Mean counter value (KiB) per kernel name over its dispatches."""
    acc = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter:
                continue
            acc.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return {k: (sum(v) / len(v), len(v)) for k, v in acc.items()}


def _short(name):
    m = re.search(r"(\w+_kernel)(<[^>]*>)?", name)
    return m.group(1) + (m.group(2) or "") if m else name[:60]


def summarize_pmc(fetch_csv, write_csv, copy_fetch_csv, copy_write_csv, out, copy_mib, command):
    """Per-launch HBM traffic of each kernel, scaled by the copy calibration."""
    fetch = _pmc_means(fetch_csv, "FETCH_SIZE")
    write = _pmc_means(write_csv, "WRITE_SIZE")
    cf = _pmc_means(copy_fetch_csv, "FETCH_SIZE")
    cw = _pmc_means(copy_write_csv, "WRITE_SIZE")
    # The copy kernel is the bf16 elementwise mul of --copy-calibration; it is
    # the one launched 5 times, reading and writing copy_mib MiB each time.
    copy_name = max((k for k in cf if cf[k][1] == 5 and k in cw), key=lambda k: cw[k][0])
    known_kib = copy_mib * 1024.0
    f_fetch = known_kib / cf[copy_name][0]
    f_write = known_kib / cw[copy_name][0]
    kernels = {}
    for name, (fk, n) in fetch.items():
        if name not in write or not name.startswith("void moe::"):
            continue
        wk = write[name][0]
        kernels[_short(name)] = {
            "fetch_kib": round(fk, 1), "write_kib": round(wk, 1), "dispatches": n,
            "traffic_bytes": int(round((fk * f_fetch + wk * f_write) * 1024))}
    units = sorted({kernel_unit(k) for k in kernels})
    summary = {"source_hashes": {u: kernel_source_hash(u) for u in units},
               "copy_kernel": copy_name[:80],
               "copy_known_kib": known_kib, "copy_fetch_kib": round(cf[copy_name][0], 1),
               "copy_write_kib": round(cw[copy_name][0], 1), "fetch_factor": round(f_fetch, 5),
               "write_factor": round(f_write, 5), "kernels": kernels, "command": command}
    with open(out, "w") as f:
        f.write("# HBM traffic per launch from rocprofv3 --pmc FETCH_SIZE and WRITE_SIZE runs,\n")
        f.write("# each counter scaled by what it reads on a plain copy kernel of known size.\n")
        f.write(json.dumps(summary, indent=1) + "\n")
    print(out)


def summarize_trace(stats_csv, out, command):
    rows = list(csv.DictReader(open(stats_csv)))
    with open(out, "w") as f:
        f.write("# rocprofv3 --kernel-trace --stats summary\n# command: %s\n" % command)
        f.write("%-60s %7s %12s %12s %12s\n" % ("kernel", "calls", "avg_us", "min_us", "max_us"))
        for r in rows:
            f.write("%-60s %7s %12.2f %12.2f %12.2f\n" % (
                r["Name"][:60], r["Calls"], float(r["AverageNs"]) / 1e3,
                float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3))
    print(out)


def recorded_traffic(workload, kernel):
    """(kernel, traffic per launch) of `kernel` in the committed summary for
    the workload, if the summary is still current."""
    path = os.path.join(PROFILES, f"hbm_traffic_{workload}.txt")
    if not os.path.exists(path):
        return None, None
    text = "".join(ln for ln in open(path) if not ln.startswith("#"))
    s = json.loads(text)
    unit = kernel_unit(kernel)
    if s.get("source_hashes", {}).get(unit) != kernel_source_hash(unit):
        return None, None
    for name, v in s["kernels"].items():
        if name.split("<")[0] == kernel:
            return name, v["traffic_bytes"]
    return None, None


def algorithmic_bytes(wl, D, payload="bf16", hier=False):
    """(dispatch, combine) payload bytes of one step."""
    row = 2 * wl.hidden
    T, k = wl.num_tokens, wl.top_k
    if hier:
        # hop 1 reads T*k rows and writes D fp32 partials; hop 2 reads them back
        return (T + 2 * D + T * k) * row, (T * k + T) * row + 2 * D * 2 * row
    if payload == "fp8":
        # token rows are read (and combine results written) as bf16; the k
        # receive rows (and the D staging rows, written once and read once)
        # carry one byte per element plus a float32 per 128 elements
        row8 = wl.hidden + 4 * ((wl.hidden + 127) // 128)
        return T * row + (2 * D + T * k) * row8, T * k * row8 + T * row
    disp = (T + T * k) * row if not wl.node_dedup else (T + 2 * D + T * k) * row
    comb = (T * k + T) * row
    return disp, comb


def kernel_bytes(wl, D, payload="bf16", chunks=None, hier_chunks=None):
    """Algorithmic payload bytes per step moved by each kernel (by symbol).

    chunks: (tokens, staging rows) of each chunk of the deduplicated dispatch,
    which launches hop 1 of chunk 0, then hop 2 of chunk c with hop 1 of
    chunk c + 1 (stage_ab), then hop 2 of the last chunk; hier_chunks: the
    same for the hierarchical combine (combine_part, combine_pn,
    combine_nodes)."""
    row = 2 * wl.hidden
    row8 = wl.hidden + 4 * ((wl.hidden + 127) // 128)
    T, k = wl.num_tokens, wl.top_k
    single = (T + T * k) * row
    out = {
        "gather_kernel": single, "gather_scan_kernel": single,
        "stage_a_kernel": (T + D) * row, "stage_b_kernel": (D + T * k) * row,
        "combine_kernel": (T * k + T) * row,
        "combine_part_kernel": T * k * row + D * 2 * row,
        "combine_nodes_kernel": D * 2 * row + T * row,
        "gather_fp8_kernel": T * row + T * k * row8, "gather_fp8_scan_kernel": T * row + T * k * row8,
        "stage_a_fp8_kernel": T * row + D * row8, "stage_b_fp8_kernel": D * row8 + T * k * row8,
        "combine_fp8_kernel": T * k * row8 + T * row,
        "pipeline_kernel": 2 * (T + T * k) * row,
    }

    def split(first_b, last_b, fused, hop1, hop2):
        out[first_b] = hop1[0]
        out[last_b] = hop2[-1]
        out[fused] = sum(hop2[:-1]) + sum(hop1[1:])

    if chunks is not None:
        tc, dc = chunks
        if payload == "fp8":
            split("stage_a_fp8_kernel", "stage_b_fp8_kernel", "stage_ab_fp8_kernel",
                  [t * row + d * row8 for t, d in zip(tc, dc)],
                  [d * row8 + t * k * row8 for t, d in zip(tc, dc)])
        else:
            split("stage_a_kernel", "stage_b_kernel", "stage_ab_kernel",
                  [(t + d) * row for t, d in zip(tc, dc)], [(d + t * k) * row for t, d in zip(tc, dc)])
    if hier_chunks is not None:
        tc, dc = hier_chunks
        split("combine_part_kernel", "combine_nodes_kernel", "combine_pn_kernel",
              [t * k * row + d * 2 * row for t, d in zip(tc, dc)],
              [d * 2 * row + t * row for t, d in zip(tc, dc)])
    return out


def cpu_baseline(batch, seconds, payload="bf16", band=0, hier=False):
    """The oracle (numpy, as it stands) timed on this host on the same batch:
    whole passes until `seconds` have been spent (at least one)."""
    import oracle
    from oracle import fp8 as ofp8

    wl = batch.workload
    reps, t0 = 0, time.perf_counter()
    D = 0
    while True:
        if band:
            p = oracle.route_plan_banded(batch.topk_idx, wl.num_experts, wl.num_ranks, band)
        else:
            p = oracle.route_plan(batch.topk_idx, wl.num_experts, wl.num_ranks, wl.ranks_per_node)
        if payload == "fp8":
            if wl.node_dedup:
                _, _, codes, exps = ofp8.dedup_dispatch_fp8(batch.x, p)
            else:
                codes, exps = ofp8.dispatch_fp8(batch.x, p)
            ofp8.combine_fp8(codes, exps, batch.topk_w, p)
        else:
            if wl.node_dedup:
                recv = oracle.dedup_stage_b(oracle.dedup_stage_a(batch.x, p), p)
            else:
                recv = oracle.dispatch(batch.x, p)
            if hier:
                oracle.combine_hierarchical(recv, batch.topk_w, p)
            else:
                oracle.combine(recv, batch.topk_w, p)
        D = p.get("num_staged", 0)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    disp, comb = algorithmic_bytes(wl, D, payload, hier)
    return {"value": round((disp + comb) * reps / el / 1e9, 4), "unit": "GB/s", "cores": 1,
            "kind": "oracle",
            "sample": f"{reps} full pass(es) of the {wl.name} batch ({payload} payload: "
                      f"{'banded ' if band else ''}route plan, dispatch, "
                      f"{'hierarchical ' if hier else ''}combine in float64) in {el:.1f} s on "
                      f"1 thread (numpy element-wise); os.cpu_count()={os.cpu_count()}, "
                      f"affinity={len(os.sched_getaffinity(0))}"}


def stats(ms):
    """Median, mean, p10 and p90 of a list of milliseconds."""
    a = np.asarray(ms, dtype=np.float64)
    q = np.percentile(a, [50, 10, 90])
    return {"ms_median": round(float(q[0]), 5), "ms_mean": round(float(a.mean()), 5),
            "ms_p10": round(float(q[1]), 5), "ms_p90": round(float(q[2]), 5)}


class Flush:
    """Evicts the last-level cache: writes a 1 GiB scratch buffer, then reads
    another 1 GiB buffer (clean lines of unrelated data in the cache)."""

    def __init__(self, torch, dev):
        n = FLUSH_BYTES // 4
        self.w = torch.empty(n, dtype=torch.int32, device=dev)
        self.r = torch.ones(n, dtype=torch.int32, device=dev)
        self.i = 0

    def __call__(self):
        self.i += 1
        self.w.fill_(self.i)
        return self.r.sum()


def run_workload(torch, cs, gen, name, args, dev, flush, primary):
    """Everything measured on one workload; returns (result dict, batch)."""
    wl = gen.get(name)
    fp8 = args.payload == "fp8"
    batch = gen.make_batch(wl)
    if args.single_hop and wl.node_dedup:
        # the same routing, planned as one node: dispatch is the single-hop gather
        wl = dataclasses.replace(wl, name=wl.name + "-single-hop", ranks_per_node=wl.num_ranks)
    T, H, k = wl.num_tokens, wl.hidden, wl.top_k
    la = args.load_aware_forwarders and wl.node_dedup
    hier = args.hier_combine and wl.node_dedup
    pipe = args.pipeline and not wl.node_dedup and not fp8
    band = args.band_tokens if pipe else 0

    x0 = torch.from_numpy(batch.x.view(np.int16)).to(dev)
    idx0 = torch.from_numpy(batch.topk_idx).to(dev)
    w0 = torch.from_numpy(batch.topk_w).to(dev)

    def new_set(x, idx, w):
        plan = cs.Plan(T, H, wl.num_experts, k, wl.num_ranks, wl.ranks_per_node, wl.node_dedup, la,
                       band)
        s = dict(plan=plan, x=x, idx=idx, w=w,
                 recv=torch.empty((plan.recv_rows, H), dtype=torch.int16, device=dev),
                 staging=(torch.empty((plan.staging_rows_max, H), dtype=torch.int16, device=dev)
                          if wl.node_dedup else None),
                 out=torch.empty((T, H), dtype=torch.bfloat16, device=dev))
        if hier:
            s["part"] = torch.empty((plan.staging_rows_max, H), dtype=torch.float32, device=dev)
        if fp8:
            s["recv"] = torch.empty((plan.recv_rows, H), dtype=torch.uint8, device=dev)
            s["scale"] = torch.empty((plan.recv_rows, plan.scale_blocks), dtype=torch.float32,
                                     device=dev)
            if wl.node_dedup:
                s["staging"] = torch.empty((plan.staging_rows_max, H), dtype=torch.uint8, device=dev)
                s["sscale"] = torch.empty((plan.staging_rows_max, plan.scale_blocks),
                                          dtype=torch.float32, device=dev)
        return s

    def do_route(s, st=None):
        s["plan"].route(s["idx"], stream=st)

    def do_dispatch(s, st=None):
        if fp8:
            s["plan"].dispatch_fp8(s["x"], s["recv"], s["scale"], s["staging"], s.get("sscale"),
                                   stream=st)
        else:
            s["plan"].dispatch(s["x"], s["recv"], s["staging"], stream=st)

    def do_combine(s, st=None):
        if hier:
            s["plan"].combine_hier(s["recv"], s["w"], s["part"], s["out"], stream=st)
        elif fp8:
            s["plan"].combine_fp8(s["recv"], s["scale"], s["w"], s["out"], stream=st)
        else:
            s["plan"].combine(s["recv"], s["w"], s["out"], stream=st)

    def phase1(s, st=None):
        if pipe:
            s["plan"].pipeline(s["idx"], s["x"], s["w"], s["recv"], s["out"], stream=st)
        else:
            do_route(s, st)
            do_dispatch(s, st)

    def step(s, st=None):
        phase1(s, st)
        if not pipe:
            do_combine(s, st)

    main = torch.cuda.current_stream(dev)
    s0 = new_set(x0, idx0, w0)

    def protocol_steps(n, flush_mid=True, timed=False):
        """n flushed steps on stream 0: flush, phase 1, flush, phase 2.

        Marker events bracket each phase.  timed: the library also times every
        launch (events bound to each kernel's own start and end), read back
        after each phase.  Returns the per-step marker times of both phases,
        each phase's span from its first kernel's start to its last kernel's
        end (timed only), and the timed launches."""
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(n)]
        kern = [[], []]
        launches = []

        def span(ls):
            launches.extend(ls)
            return max(st + ms for _, st, ms in ls) - min(st for _, st, _ in ls)

        for i in range(n):
            ev = evs[i]
            flush()
            ev[0].record()
            phase1(s0)
            ev[1].record()
            if timed:
                kern[0].append(span(s0["plan"].timing_read()))
            if not pipe:
                if flush_mid:
                    flush()
                ev[2].record()
                do_combine(s0)
                ev[3].record()
                if timed:
                    kern[1].append(span(s0["plan"].timing_read()))
        torch.cuda.synchronize()
        p1 = [e[0].elapsed_time(e[1]) for e in evs]
        p2 = [] if pipe else [e[2].elapsed_time(e[3]) for e in evs]
        return p1, p2, kern[0], kern[1], launches

    # Warmup, in the protocol's own flushed form.
    protocol_steps(max(1, args.warmup))
    D = int(s0["plan"].read("num_staged")[0]) if wl.node_dedup else 0
    fwd_rows = None
    if wl.node_dedup:
        per = np.diff(s0["plan"].read("stage_offsets"))
        fwd_rows = {"rule": "load_aware" if la else "static", "max": int(per.max()),
                    "mean": round(float(per.mean()), 1),
                    "max_over_mean": round(float(per.max() / max(per.mean(), 1e-9)), 4)}
    disp_b, comb_b = algorithmic_bytes(wl, D, args.payload, hier)
    step_b = disp_b + comb_b

    # The timed region: exactly K flushed steps, bracketed by synchronize,
    # each phase between two hipEventRecord markers on the step's stream.
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    p1, p2, _, _, _ = protocol_steps(args.steps)
    wall_ms = (time.perf_counter() - t0) * 1e3 / args.steps

    # Kernel pass: K more flushed steps with every launch timed by the
    # library.  Binding events to a launch adds a gap of a few microseconds
    # after it, so this pass gives kernel durations, not phase times.
    s0["plan"].timing(256)
    launches = protocol_steps(args.steps, timed=True)[4]
    s0["plan"].timing(0)

    def phase_stats(marker, nbytes):
        st = stats(marker)
        return {"bytes": nbytes, **st, "GB/s": round(nbytes / (st["ms_median"] * 1e-3) / 1e9, 1)}

    if pipe:
        phases = {"pipeline": phase_stats(p1, step_b)}
        ms_step = phases["pipeline"]["ms_median"]
    else:
        phases = {"route_dispatch": phase_stats(p1, disp_b), "combine": phase_stats(p2, comb_b)}
        ms_step = phases["route_dispatch"]["ms_median"] + phases["combine"]["ms_median"]
    value = step_b / (ms_step * 1e-3) / 1e9
    res = {"value": round(value, 2), "ms_per_step": round(ms_step, 5),
           "pct_of_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
           "bytes_per_step": step_b,
           "config": {"workload": wl.name, "T": T, "H": H, "E": wl.num_experts, "k": k,
                      "R": wl.num_ranks, "G": wl.ranks_per_node, "node_dedup": wl.node_dedup,
                      "staging_rows": D, "seed": wl.seed, "payload": args.payload,
                      "forwarder_rows": fwd_rows,
                      "combine": "hierarchical" if hier else "direct",
                      "path": f"pipeline, bands of {band} tokens" if pipe else "separate launches"},
           "protocol": {"flush": "1 GiB written, then another 1 GiB read, before each phase "
                                 "(not timed)",
                        "phase_time": "hipEventRecord markers around each phase on the step's "
                                      "stream; an interval also holds the launch latency of the "
                                      "phase's first kernel (not subtracted)",
                        "phases": phases,
                        "wall_ms_per_step_incl_flush": round(wall_ms, 5)}}
    if not pipe and wl.name.startswith("olmoe") and not args.no_schedules:
        # The receive rows (128 MiB) fit the MALL: the combine without the
        # flush between the phases, for comparison.
        _, p2r, _, _, _ = protocol_steps(args.steps, flush_mid=False)
        r = stats(p2r)
        res["protocol"]["combine_mall_resident"] = {
            **r, "GB/s": round(comb_b / (r["ms_median"] * 1e-3) / 1e9, 1),
            "note": "no flush between dispatch and combine: the receive rows stay in the MALL"}

    # Every kernel's launches in the timed steps.
    chunks = hier_chunks = None
    if wl.node_dedup:
        src = s0["plan"].read("stage_src")[:D]

        def per_chunk(n):
            """(tokens, staging rows) of each chunk of n tokens."""
            nch = -(-T // n)
            return ([min(T, (c + 1) * n) - c * n for c in range(nch)],
                    np.bincount(src // n, minlength=nch).tolist())

        chunks = per_chunk(s0["plan"].chunk_tokens["dispatch_fp8" if fp8 else "dispatch"])
        if hier:
            hier_chunks = per_chunk(s0["plan"].chunk_tokens["combine_hier"])
    kb = kernel_bytes(wl, D, args.payload, chunks, hier_chunks)
    agg = {}
    for kname, _, ms in launches:
        a = agg.setdefault(kname, [0, 0.0])
        a[0] += 1
        a[1] += ms
    kernels = {}
    for kname, (n, tot) in agg.items():
        e = {"launches_per_step": round(n / args.steps, 3), "avg_us": round(1e3 * tot / n, 3),
             "us_per_step": round(1e3 * tot / args.steps, 3)}
        if kname in kb:
            gbs = kb[kname] / (tot / args.steps * 1e-3) / 1e9
            e.update({"bytes_per_step": kb[kname], "GB/s": round(gbs, 1),
                      "frac": round(gbs / HBM_PEAK_GBS, 4)})
        kernels[kname] = e
    res["kernels"] = kernels
    ksum = sum(e["us_per_step"] for e in kernels.values()) * 1e-3
    res["kernel_time_per_step"] = {
        "ms": round(ksum, 5), "value": round(step_b / (ksum * 1e-3) / 1e9, 2),
        "note": "sum of every kernel's mean duration per step (no launch gaps)"}
    moving = [kn for kn in kernels if kn in kb]
    dom = max(moving, key=lambda kn: kernels[kn]["us_per_step"])
    dk = kernels[dom]
    per_launch_b = kb[dom] / dk["launches_per_step"]
    variant = ("_pipeline" if pipe else "_fp8" if fp8 else "_hier" if hier else
               "_single_hop" if wl.name.endswith("-single-hop") else "")
    traffic_kernel, traffic = recorded_traffic(name + variant, dom)
    res["roofline"] = {"bound": "hbm", "kernel": traffic_kernel or dom, "achieved": dk["GB/s"],
                       "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": dk["frac"],
                       "traffic": traffic,
                       "traffic_over_algorithmic": (None if traffic is None else
                                                    round(traffic / per_launch_b, 4)),
                       "bytes_per_launch": int(round(per_launch_b)), "us_per_launch": dk["avg_us"],
                       "launches_per_step": dk["launches_per_step"],
                       "timing": "HIP events bound to each launch (moe_plan_timing) in the "
                                 "timed steps"}

    if not args.no_schedules:
        res["schedules"] = schedules(torch, wl, args, dev, x0, idx0, w0, new_set, do_route,
                                     do_dispatch, do_combine, step, pipe, step_b)
        res["copy_ceiling"] = copy_ceiling(torch, dev, step_b // 2, args.steps)
        res["copy_ceiling"]["value_over_copy"] = round(value / res["copy_ceiling"]["GB/s"], 4)
    del s0
    torch.cuda.empty_cache()
    return res, batch, hier, band


def schedules(torch, wl, args, dev, x0, idx0, w0, new_set, do_route, do_dispatch, do_combine,
              step, pipe, step_b):
    """Back-to-back steps (no flush) in four schedules over cycled buffer sets."""
    set_b = (x0.numel() * 2 + idx0.numel() * 4 + w0.numel() * 4)
    probe = new_set(x0, idx0, w0)
    full_b = set_b + sum(t.numel() * t.element_size() for key, t in probe.items()
                         if key in ("recv", "staging", "out", "part", "scale", "sscale")
                         and t is not None) + probe["plan"].workspace_bytes
    del probe
    max_inflight = 1 if pipe else 2
    n_sets = args.sets or min(MAX_SETS, max(2, math.ceil((2 << 30) / full_b),
                                            math.ceil(4 * MALL_BYTES / set_b)))
    n_sets = -(-n_sets // max_inflight) * max_inflight
    sets = [new_set(x0.clone(), idx0.clone(), w0.clone()) for _ in range(n_sets)]
    streams = [torch.cuda.current_stream(dev)] + [torch.cuda.Stream(dev)
                                                  for _ in range(max_inflight - 1)]

    def staggered_step(i, done):
        s, st = sets[i % n_sets], streams[i % 2]
        do_route(s, st)
        if i > 0:
            st.wait_event(done[(i - 1) % 2])
        do_dispatch(s, st)
        done[i % 2].record(st)
        do_combine(s, st)

    def plan_ahead_steps(steps):
        main, side = streams[0], streams[1]
        routed = [torch.cuda.Event(), torch.cuda.Event()]
        moving = torch.cuda.Event()
        do_route(sets[0], side)
        routed[0].record(side)
        for i in range(steps):
            s = sets[i % n_sets]
            main.wait_event(routed[i % 2])
            moving.record(main)
            do_dispatch(s, main)
            do_combine(s, main)
            if i + 1 < steps:
                s1 = sets[(i + 1) % n_sets]
                side.wait_event(moving)
                do_route(s1, side)
                routed[(i + 1) % 2].record(side)

    def timed(schedule, steps):
        done = [torch.cuda.Event(), torch.cuda.Event()]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        if schedule == "plan_ahead":
            plan_ahead_steps(steps)
        else:
            for i in range(steps):
                if schedule == "staggered":
                    staggered_step(i, done)
                else:
                    step(sets[i % n_sets], streams[i % (2 if schedule == "two_in_flight" else 1)])
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / steps

    for i in range(max(args.warmup, n_sets)):
        step(sets[i % n_sets], streams[i % max_inflight])
    names = SCHEDULES if max_inflight == 2 else ("serial",)
    out = {"buffer_sets": n_sets}
    for nm in names:
        ms = timed(nm, args.steps)
        v = step_b / (ms * 1e-3) / 1e9
        out[nm] = {"ms_per_step": round(ms, 5), "value": round(v, 2),
                   "pct_of_hbm_peak": round(100.0 * v / HBM_PEAK_GBS, 2)}
    out["best"] = min(names, key=lambda nm: out[nm]["ms_per_step"])
    del sets
    torch.cuda.empty_cache()
    return out


def main():
    args = parse()
    if args.summarize_trace:
        summarize_trace(*args.summarize_trace, args.command)
        return
    if args.summarize_pmc:
        summarize_pmc(*args.summarize_pmc, args.copy_mib, args.command)
        return
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the expert-parallel ranks are virtual "
              f"partitions of a single MI355X's HBM; --gpus {args.gpus} is not supported.",
              file=sys.stderr)
        sys.exit(2)
    if args.hier_combine and args.payload == "fp8":
        print("the hierarchical combine takes the bf16 payload", file=sys.stderr)
        sys.exit(2)

    import torch

    import combine_shuffling_amd as cs
    from workloads import gen

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    flush = Flush(torch, dev)
    head, batch, hier, band = run_workload(torch, cs, gen, args.workload, args, dev, flush, True)
    print(f"# {args.workload}: {head['value']} GB/s ({head['pct_of_hbm_peak']}%)", file=sys.stderr,
          flush=True)
    per_config = {}
    extra = [] if args.configs in ("", "none") else args.configs.split(",")
    for nm in extra:
        if nm == args.workload:
            continue
        r, _, _, _ = run_workload(torch, cs, gen, nm, args, dev, flush, False)
        per_config[nm] = r
        print(f"# {nm}: {r['value']} GB/s ({r['pct_of_hbm_peak']}%)", file=sys.stderr, flush=True)

    result = {
        "metric": METRIC,
        "value": head["value"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": args.payload,
        "data": "synthetic",
        "config": head["config"],
        "pct_of_hbm_peak": head["pct_of_hbm_peak"],
        "bytes_per_step": head["bytes_per_step"],
        "protocol": head["protocol"],
        "roofline": head["roofline"],
        "kernels": head["kernels"],
        "kernel_time_per_step": head["kernel_time_per_step"],
        "schedules": head.get("schedules"),
        "copy_ceiling": head.get("copy_ceiling"),
        "per_config": per_config,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(batch, args.cpu_seconds, args.payload, band, hier)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
