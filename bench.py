"""Benchmark: MoE expert-parallel shuffle (route plan + dispatch + combine) on one MI355X.

One step = one pass of the whole path over one batch: moe_route_plan (histogram,
scan, segment descriptors), moe_dispatch (single hop, or the two hops of node
deduplication for the DeepSeek-V3-like workload) and moe_combine (bf16 out),
with the identity expert between dispatch and combine.

Inputs are resident in HBM before timing starts, and no step finds them in
a cache.  Consecutive steps cycle through independent copies of every buffer
(inputs, plan workspace, receive and staging rows, outputs).  The rows are
streamed with non-temporal accesses, which leave the 256 MB last-level cache
(MALL) to what is read with plain loads, the token rows x above all; so the
copies of the inputs total at least four times the MALL (and the copies of
everything at least 2 GiB), and each step reads its x from HBM.  With fewer
copies the MALL keeps x between steps: on the non-divisible workload, x
cycled over 2 copies (268 MB) gives a 164 us dispatch, over 4 copies 183 us,
and one copy reused 151 us.  Within a step combine reads the rows dispatch
has just written, as the path does.

Prints one JSON line.
  value       algorithmic payload bytes per step / wall time per step, over K
              steps bracketed by synchronize on both sides, no timing events
              inside.  Schedule (--inflight auto): after the warmup, a short
              trial of four schedules picks the fastest: serial (the steps
              one after another on one stream), two_in_flight (step i on
              stream i mod 2, each stream in order), staggered (as
              two_in_flight, with each step's dispatch waiting on an event
              after the previous step's dispatch, so a dispatch always runs
              beside the other batch's combine) and plan_ahead (dispatch and
              combine on one stream, each step's route plan on a second
              stream while the previous step moves its rows).  The K timed steps run in the
              chosen one; K steps of each other schedule are timed too and
              reported beside it.
  phases      route plan, dispatch and combine timed inside K more steps
              run one after another on one stream, with HIP events on that
              stream between the phases.  Inside a step, the non-temporal
              writes a kernel leaves behind drain while the next kernel runs,
              so each phase is timed in the order the step runs it (timed
              alone, back to back, the same kernels measured the other way
              round: qwen3 gather 117 us alone vs 93 us in a step, combine
              104 vs 116 us).  An event exposes one kernel-launch latency
              (about 2.5 us) that back-to-back kernels hide: the phase times
              have it subtracted, estimated as (sum of the phase intervals -
              the serial step time) / 3.  The value pass has no events.
              Each phase also gives its median, p10 and p90 over the K steps.
  roofline    the dominant kernel: its algorithmic bytes per launch / its mean
              duration from the phase pass.
              traffic = HBM bytes per launch from the rocprofv3 FETCH_SIZE /
              WRITE_SIZE summary under profiles/, scaled by the copy
              calibration; null if the kernel sources changed since.
              traffic_over_algorithmic: above 1 means bytes moved twice.
  copy_ceiling a plain device-to-device copy (torch copy_) moving the step's
              bytes, half read and half written, over source/destination
              pairs cycled past the MALL, K times: a practical ceiling, and
              value over it.
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
MAX_SETS = 256
METRIC = "dispatch+combine effective GB/s and % of HBM peak, 1 MI355X"
SCHEDULES = ("serial", "two_in_flight", "staggered", "plan_ahead")
PROFILES = os.path.join(ROOT, "profiles")
KERNEL_SOURCES = ("combine_shuffling_amd/csrc/move.hip", "combine_shuffling_amd/csrc/move_body.h",
                  "combine_shuffling_amd/csrc/pipeline.hip", "combine_shuffling_amd/csrc/plan_body.h",
                  "combine_shuffling_amd/csrc/moe_device.h",
                  "combine_shuffling_amd/csrc/moe_internal.h")


def parse():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="olmoe",
                    help="tiny | olmoe | qwen3 | dsv3 | nondiv (default: olmoe, the OLMoE-like prefill)")
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
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--sets", type=int, default=0, help="buffer sets to cycle (0: auto)")
    ap.add_argument("--inflight", default="auto", choices=("auto", "1", "2", "staggered", "plan_ahead"),
                    help="schedule of the steps.  1: one stream, every step after the previous "
                         "one.  2: two batches in flight, step i on HIP stream i mod 2, each "
                         "stream running its steps in order.  staggered: as 2, but each step's "
                         "dispatch waits for the previous step's dispatch, so a dispatch always "
                         "overlaps the other batch's combine.  plan_ahead: dispatch and combine "
                         "on one stream, each step's route plan on a second stream during the "
                         "previous step's movement.  auto (default): a short trial of the four "
                         "after the warmup picks the fastest for the timed steps")
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
    return ap.parse_args()


def kernel_source_hash():
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
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
    summary = {"source_hash": kernel_source_hash(), "copy_kernel": copy_name[:80],
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


def recorded_traffic(workload, kernels):
    """(kernel, traffic per launch) of the first of `kernels` (names separated by
    '|') in the committed summary, if the summary is still current."""
    path = os.path.join(PROFILES, f"hbm_traffic_{workload}.txt")
    if not os.path.exists(path):
        return None, None
    text = "".join(ln for ln in open(path) if not ln.startswith("#"))
    s = json.loads(text)
    if s.get("source_hash") != kernel_source_hash():
        return None, None
    for kernel in kernels.split("|"):
        for name, v in s["kernels"].items():
            if name.split("<")[0] == kernel:
                return name, v["traffic_bytes"]
    return None, None


def algorithmic_bytes(wl, D, payload="bf16", hier=False):
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


def cpu_baseline(batch, seconds, payload="bf16", band=0):
    """The oracle (numpy, as it stands) timed on this host on the same batch."""
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
            oracle.combine(recv, batch.topk_w, p)
        D = p.get("num_staged", 0)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    disp, comb = algorithmic_bytes(wl, D, payload)
    return {"value": round((disp + comb) * reps / el / 1e9, 4), "unit": "GB/s", "cores": 1,
            "kind": "oracle",
            "sample": f"{reps} full passes of the {wl.name} batch ({payload} payload: "
                      f"{'banded ' if band else ''}route plan, dispatch, combine in float64) "
                      f"in {el:.1f} s on 1 thread; "
                      f"os.cpu_count()={os.cpu_count()}, affinity={len(os.sched_getaffinity(0))}"}


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

    import torch

    import combine_shuffling_amd as cs
    from workloads import gen

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    wl = gen.get(args.workload)
    fp8 = args.payload == "fp8"
    batch = gen.make_batch(wl)
    if args.single_hop and wl.node_dedup:
        # the same routing, planned as one node: dispatch is the single-hop gather
        wl = dataclasses.replace(wl, name=wl.name + "-single-hop", ranks_per_node=wl.num_ranks)
    T, H, k = wl.num_tokens, wl.hidden, wl.top_k

    x0 = torch.from_numpy(batch.x.view(np.int16)).to(dev)
    idx0 = torch.from_numpy(batch.topk_idx).to(dev)
    w0 = torch.from_numpy(batch.topk_w).to(dev)

    la = args.load_aware_forwarders and wl.node_dedup
    hier = args.hier_combine and wl.node_dedup
    if hier and fp8:
        print("the hierarchical combine takes the bf16 payload", file=sys.stderr)
        sys.exit(2)
    pipe = args.pipeline
    if pipe and (wl.node_dedup or fp8):
        print("the banded pipeline runs single-hop workloads with the bf16 payload",
              file=sys.stderr)
        sys.exit(2)
    band = args.band_tokens if pipe else 0
    probe = cs.Plan(T, H, wl.num_experts, k, wl.num_ranks, wl.ranks_per_node, wl.node_dedup, la,
                    band)
    set_bytes = (x0.numel() * 2 + idx0.numel() * 4 + w0.numel() * 4 + probe.workspace_bytes
                 + probe.recv_rows * H * (1 if fp8 else 2) + probe.staging_rows_max * H * 2
                 + T * H * 2)
    in_bytes = x0.numel() * 2 + idx0.numel() * 4 + w0.numel() * 4
    auto = str(args.inflight) == "auto"
    max_inflight = 1 if pipe or args.inflight == "1" else 2
    n_sets = args.sets or min(MAX_SETS, max(2, math.ceil((2 << 30) / set_bytes),
                                            math.ceil(4 * MALL_BYTES / in_bytes)))
    # a set always runs on the same stream, so its reuse is ordered after its last use
    n_sets = -(-n_sets // max_inflight) * max_inflight
    sets = []
    for _ in range(n_sets):
        plan = cs.Plan(T, H, wl.num_experts, k, wl.num_ranks, wl.ranks_per_node, wl.node_dedup, la,
                       band)
        s = dict(plan=plan, x=x0.clone(), idx=idx0.clone(), w=w0.clone(),
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
        sets.append(s)

    # Stream 0 is torch's current stream; the others are plain streams of the
    # default priority.
    streams = [torch.cuda.current_stream(dev)] + [torch.cuda.Stream(dev)
                                                  for _ in range(max_inflight - 1)]

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

    def step(s, st=None):
        if pipe:
            s["plan"].pipeline(s["idx"], s["x"], s["w"], s["recv"], s["out"], stream=st)
            return
        s["plan"].route(s["idx"], stream=st)
        do_dispatch(s, st)
        do_combine(s, st)

    def staggered_step(i, done):
        """Step i on stream i % 2, its dispatch after step i - 1's dispatch
        (event done[i - 1]), so that it overlaps step i - 1's combine."""
        s, st = sets[i % n_sets], streams[i % 2]
        s["plan"].route(s["idx"], stream=st)
        if i > 0:
            st.wait_event(done[(i - 1) % 2])
        do_dispatch(s, st)
        done[i % 2].record(st)
        do_combine(s, st)

    def plan_ahead_steps(steps):
        """Step i's dispatch and combine on stream 0; its route plan on
        stream 1, during step i - 1's dispatch and combine (the event moving
        orders it after step i - 2, the last user of its buffer set)."""
        main, side = streams[0], streams[1]
        routed = [torch.cuda.Event(), torch.cuda.Event()]
        moving = torch.cuda.Event()
        sets[0]["plan"].route(sets[0]["idx"], stream=side)
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
                s1["plan"].route(s1["idx"], stream=side)
                routed[(i + 1) % 2].record(side)

    def timed_steps(schedule, steps=None):
        """Wall time per step of K steps in one schedule: "serial" (one
        stream), "two_in_flight" (step i on stream i % 2), "staggered" or
        "plan_ahead"."""
        steps = args.steps if steps is None else steps
        done = [torch.cuda.Event(), torch.cuda.Event()]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        if schedule == "plan_ahead":
            plan_ahead_steps(steps)
        for i in range(steps if schedule != "plan_ahead" else 0):
            if schedule == "staggered":
                staggered_step(i, done)
            else:
                step(sets[i % n_sets], streams[i % (2 if schedule == "two_in_flight" else 1)])
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / steps

    for i in range(args.warmup):
        step(sets[i % n_sets], streams[i % max_inflight])
    torch.cuda.synchronize()
    # Schedule: a trial of each, apart from the timed steps, picks the fastest.
    trial = None
    if max_inflight == 1:
        schedule = "serial"
    elif auto:
        n_trial = max(20, args.steps // 4)
        trial = {name: timed_steps(name, n_trial) for name in SCHEDULES}
        schedule = min(trial, key=trial.get)
    else:
        schedule = {"2": "two_in_flight"}.get(args.inflight, args.inflight)
    inflight = 1 if schedule == "serial" else 2
    D = int(sets[0]["plan"].read("num_staged")[0]) if wl.node_dedup else 0
    fwd_rows = None
    if wl.node_dedup:
        per = np.diff(sets[0]["plan"].read("stage_offsets"))
        fwd_rows = {"rule": "load_aware" if la else "static", "max": int(per.max()),
                    "mean": round(float(per.mean()), 1),
                    "max_over_mean": round(float(per.max() / max(per.mean(), 1e-9)), 4)}
    disp_b, comb_b = algorithmic_bytes(wl, D, args.payload, hier)

    # Timed region: K steps and nothing else, with `inflight` batches in
    # flight; then K steps of the other schedule, reported beside it.
    ms_per_step = timed_steps(schedule)
    value = (disp_b + comb_b) / (ms_per_step * 1e-3) / 1e9
    per_schedule = {schedule: ms_per_step}
    for name in (SCHEDULES if max_inflight == 2 else ("serial",)):
        if name not in per_schedule:
            per_schedule[name] = timed_steps(name)
    serial_ms = per_schedule["serial"]
    serial_value = (disp_b + comb_b) / (serial_ms * 1e-3) / 1e9

    def schedule_entry(name):
        if name not in per_schedule:
            return None
        v = (disp_b + comb_b) / (per_schedule[name] * 1e-3) / 1e9
        return {"ms_per_step": round(per_schedule[name], 5), "value": round(v, 2),
                "pct_of_hbm_peak": round(100.0 * v / HBM_PEAK_GBS, 2)}

    # Phase pass: K more steps one after another on stream 0, with events
    # between the phases (route plan | dispatch | combine).
    def phase_pass():
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
        torch.cuda.synchronize()
        for i in range(args.steps):
            s, ev = sets[i % n_sets], evs[i]
            ev[0].record()
            if pipe:
                step(s)
                ev[1].record()
                ev[2].record()
            else:
                s["plan"].route(s["idx"])
                ev[1].record()
                do_dispatch(s)
                ev[2].record()
                do_combine(s)
            ev[3].record()
        torch.cuda.synchronize()
        return np.array([[e[0].elapsed_time(e[1]), e[1].elapsed_time(e[2]),
                          e[2].elapsed_time(e[3])] for e in evs])

    phase_t = phase_pass()
    route_ms, disp_ms, comb_ms = (float(v) for v in phase_t.mean(axis=0))
    # An event makes the GPU finish the kernel before it and only then launch
    # the next one, so each interval also holds one kernel-launch latency
    # that back-to-back kernels hide.  The same steps without events (the
    # serial timing above) give it: (sum of intervals - step) / intervals.
    intervals = 1 if pipe else 3
    event_gap_ms = max(0.0, ((route_ms + disp_ms + comb_ms) if not pipe else route_ms) - serial_ms)
    event_gap_ms /= intervals
    route_ms -= event_gap_ms
    disp_ms -= event_gap_ms
    comb_ms -= event_gap_ms
    phase_t = phase_t - event_gap_ms

    def spread(col):
        """Median, p10 and p90 over the K steps of one phase (event gap removed)."""
        q = np.percentile(phase_t[:, col], [50, 10, 90])
        return {"ms_median": round(float(q[0]), 5), "ms_p10": round(float(q[1]), 5),
                "ms_p90": round(float(q[2]), 5)}
    if pipe:
        # one launch per step does everything
        pipe_ms = route_ms
        disp_ms = comb_ms = pipe_ms
        disp_gbs = comb_gbs = (disp_b + comb_b) / (pipe_ms * 1e-3) / 1e9
    else:
        disp_gbs = disp_b / (disp_ms * 1e-3) / 1e9
        comb_gbs = comb_b / (comb_ms * 1e-3) / 1e9
    if pipe:
        dom = ("pipeline_kernel", disp_b + comb_b, pipe_ms, disp_gbs)
    elif hier:
        # both phases are two launches here; report the combine phase
        dom = ("combine_part_kernel+combine_nodes_kernel", comb_b, comb_ms, comb_gbs)
    elif wl.node_dedup:
        # dispatch is two launches here; the dominant single launch timed is combine
        dom = ("combine_fp8_kernel" if fp8 else "combine_kernel", comb_b, comb_ms, comb_gbs)
    else:
        sfx = "_fp8" if fp8 else ""
        # small single-hop plans scan inside the gather (gather_scan_kernel)
        gname = "gather_fp8_scan_kernel|gather_fp8_kernel" if fp8 else "gather_scan_kernel|gather_kernel"
        dom = max([(gname, disp_b, disp_ms, disp_gbs),
                   (f"combine{sfx}_kernel", comb_b, comb_ms, comb_gbs)], key=lambda d: d[2])

    # Practical ceiling: a plain device-to-device copy moving the step's bytes
    # (half read, half written), its sources and destinations cycled past the
    # MALL like the step's buffers.
    copy = copy_ceiling(torch, dev, (disp_b + comb_b) // 2, args.steps)
    copy["value_over_copy"] = round(value / copy["GB/s"], 4)

    # which committed traffic summary covers this run
    variant = ("_pipeline" if pipe else "_fp8" if fp8 else "_hier" if hier else
               "_single_hop" if wl.name.endswith("-single-hop") else "")
    traffic_kernel, traffic = recorded_traffic(args.workload + variant, dom[0])
    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": args.payload,
        "data": "synthetic",
        "config": {"workload": wl.name, "T": T, "H": H, "E": wl.num_experts, "k": k,
                   "R": wl.num_ranks, "G": wl.ranks_per_node, "node_dedup": wl.node_dedup,
                   "staging_rows": D, "seed": wl.seed, "buffer_sets": n_sets,
                   "payload": args.payload, "forwarder_rows": fwd_rows,
                   "combine": "hierarchical" if hier else "direct",
                   "path": f"pipeline, bands of {band} tokens" if pipe else "separate launches",
                   "batches_in_flight": inflight,
                   "schedule": schedule,
                   "schedule_choice": "trial" if trial else "fixed"},
        "serial": {"ms_per_step": round(serial_ms, 5), "value": round(serial_value, 2),
                   "pct_of_hbm_peak": round(100.0 * serial_value / HBM_PEAK_GBS, 2)},
        "two_in_flight": schedule_entry("two_in_flight"),
        "staggered": schedule_entry("staggered"),
        "plan_ahead": schedule_entry("plan_ahead"),
        "schedule_trial_ms_per_step": (None if trial is None else
                                       {k2: round(v2, 5) for k2, v2 in trial.items()}),
        "pct_of_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "bytes_per_step": disp_b + comb_b,
        "phases": ({"pipeline": {"bytes": disp_b + comb_b, "ms_per_launch": round(pipe_ms, 5),
                                 "GB/s": round(disp_gbs, 1), "launches": 1}} if pipe else
                   {"route": {"ms_per_step": round(route_ms, 5), **spread(0)},
                    "dispatch": {"bytes": disp_b, "ms_per_launch": round(disp_ms, 5),
                                 "GB/s": round(disp_gbs, 1), "launches": 2 if wl.node_dedup else 1,
                                 **spread(1)},
                    "combine": {"bytes": comb_b, "ms_per_launch": round(comb_ms, 5),
                                "GB/s": round(comb_gbs, 1), "launches": 2 if hier else 1,
                                **spread(2)}}),
        "copy_ceiling": copy,
        "roofline": {"bound": "hbm", "kernel": traffic_kernel or dom[0], "achieved": round(dom[3], 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(dom[3] / HBM_PEAK_GBS, 4),
                     "traffic": traffic,
                     "traffic_over_algorithmic": (None if traffic is None or not dom[1] else
                                                  round(traffic / dom[1], 4)),
                     "bytes_per_launch": dom[1], "ms_per_launch": round(float(dom[2]), 5),
                     "event_gap_ms": round(event_gap_ms, 5)},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(batch, args.cpu_seconds, args.payload, band)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
