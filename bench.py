"""Benchmark: MoE expert-parallel shuffle (route plan + dispatch + combine) on one MI355X.

One step = one pass of the whole path over one batch: moe_route_plan (histogram,
scan, segment descriptors), moe_dispatch (single hop, or the two hops of node
deduplication for the DeepSeek-V3-like workload) and moe_combine (bf16 out),
with the identity expert between dispatch and combine.

Inputs are resident in HBM before timing starts.  Consecutive steps cycle
through several independent copies of every buffer (inputs, plan workspace,
outputs), at least 2 GiB in all, so that a step never finds the previous
step's data in the 256 MB last-level cache; within a step combine reads the
rows dispatch has just written, as the path does.

Prints one JSON line.  value = algorithmic payload bytes per step / wall time
per step (bracketed by synchronize on both sides).  Algorithmic bytes:
  dispatch single hop  (T + T*k) * 2H
  dispatch with dedup  (T + 2D + T*k) * 2H   (D staging rows, from the plan)
  combine              (T*k + T) * 2H
roofline: the dominant kernel's algorithmic bytes per launch / its mean
duration from HIP events recorded around its launch on the stream it runs on,
against the 8 TB/s HBM peak.
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "dispatch+combine effective GB/s and % of HBM peak, 1 MI355X"


def parse():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="olmoe",
                    help="tiny | olmoe | qwen3 | dsv3 | nondiv (default: olmoe, the OLMoE-like prefill)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--sets", type=int, default=0, help="buffer sets to cycle (0: auto)")
    return ap.parse_args()


def algorithmic_bytes(wl, D):
    row = 2 * wl.hidden
    T, k = wl.num_tokens, wl.top_k
    disp = (T + T * k) * row if not wl.node_dedup else (T + 2 * D + T * k) * row
    comb = (T * k + T) * row
    return disp, comb


def cpu_baseline(batch, seconds):
    """The oracle (numpy, as it stands) timed on this host on the same batch."""
    import oracle

    wl = batch.workload
    reps, t0 = 0, time.perf_counter()
    D = 0
    while True:
        p = oracle.route_plan(batch.topk_idx, wl.num_experts, wl.num_ranks, wl.ranks_per_node)
        if wl.node_dedup:
            recv = oracle.dedup_stage_b(oracle.dedup_stage_a(batch.x, p), p)
        else:
            recv = oracle.dispatch(batch.x, p)
        oracle.combine(recv, batch.topk_w, p)
        D = p["num_staged"]
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    disp, comb = algorithmic_bytes(wl, D)
    return {"value": round((disp + comb) * reps / el / 1e9, 4), "unit": "GB/s", "cores": 1,
            "kind": "oracle",
            "sample": f"{reps} full passes of the {wl.name} batch (route plan, dispatch, "
                      f"combine in float64) in {el:.1f} s on 1 thread; "
                      f"os.cpu_count()={os.cpu_count()}, affinity={len(os.sched_getaffinity(0))}"}


def main():
    args = parse()
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
    batch = gen.make_batch(wl)
    T, H, k = wl.num_tokens, wl.hidden, wl.top_k

    x0 = torch.from_numpy(batch.x.view(np.int16)).to(dev)
    idx0 = torch.from_numpy(batch.topk_idx).to(dev)
    w0 = torch.from_numpy(batch.topk_w).to(dev)

    probe = cs.Plan(T, H, wl.num_experts, k, wl.num_ranks, wl.ranks_per_node, wl.node_dedup)
    set_bytes = (x0.numel() * 2 + idx0.numel() * 4 + w0.numel() * 4 + probe.workspace_bytes
                 + probe.recv_rows * H * 2 + probe.staging_rows_max * H * 2 + T * H * 2)
    n_sets = args.sets or max(2, math.ceil((2 << 30) / set_bytes))
    sets = []
    for _ in range(n_sets):
        plan = cs.Plan(T, H, wl.num_experts, k, wl.num_ranks, wl.ranks_per_node, wl.node_dedup)
        s = dict(plan=plan, x=x0.clone(), idx=idx0.clone(), w=w0.clone(),
                 recv=torch.empty((plan.recv_rows, H), dtype=torch.int16, device=dev),
                 staging=(torch.empty((plan.staging_rows_max, H), dtype=torch.int16, device=dev)
                          if wl.node_dedup else None),
                 out=torch.empty((T, H), dtype=torch.bfloat16, device=dev))
        sets.append(s)

    def step(s, ev=None):
        s["plan"].route(s["idx"])
        if ev is not None:
            ev[0].record()
        s["plan"].dispatch(s["x"], s["recv"], s["staging"])
        if ev is not None:
            ev[1].record()
        s["plan"].combine(s["recv"], s["w"], s["out"])
        if ev is not None:
            ev[2].record()

    for i in range(args.warmup):
        step(sets[i % n_sets])
    torch.cuda.synchronize()
    D = int(sets[0]["plan"].read("num_staged")[0]) if wl.node_dedup else 0
    disp_b, comb_b = algorithmic_bytes(wl, D)

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(sets[i % n_sets], evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    disp_ms = np.array([e[0].elapsed_time(e[1]) for e in evs])
    comb_ms = np.array([e[1].elapsed_time(e[2]) for e in evs])
    ms_per_step = wall * 1e3 / args.steps
    value = (disp_b + comb_b) / (ms_per_step * 1e-3) / 1e9

    disp_gbs = disp_b / (disp_ms.mean() * 1e-3) / 1e9
    comb_gbs = comb_b / (comb_ms.mean() * 1e-3) / 1e9
    if wl.node_dedup:
        # two launches in dispatch: the dominant single kernel is combine
        dom = ("combine_kernel", comb_b, comb_ms.mean(), comb_gbs)
    else:
        dom = max([("gather_kernel", disp_b, disp_ms.mean(), disp_gbs),
                   ("combine_kernel", comb_b, comb_ms.mean(), comb_gbs)], key=lambda d: d[2])

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
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "T": T, "H": H, "E": wl.num_experts, "k": k,
                   "R": wl.num_ranks, "G": wl.ranks_per_node, "node_dedup": wl.node_dedup,
                   "staging_rows": D, "seed": wl.seed, "buffer_sets": n_sets},
        "pct_of_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "bytes_per_step": disp_b + comb_b,
        "phases": {
            "dispatch": {"bytes": disp_b, "ms_mean": round(float(disp_ms.mean()), 5),
                         "ms_p10": round(float(np.percentile(disp_ms, 10)), 5),
                         "ms_p90": round(float(np.percentile(disp_ms, 90)), 5),
                         "GB/s": round(disp_gbs, 1)},
            "combine": {"bytes": comb_b, "ms_mean": round(float(comb_ms.mean()), 5),
                        "ms_p10": round(float(np.percentile(comb_ms, 10)), 5),
                        "ms_p90": round(float(np.percentile(comb_ms, 90)), 5),
                        "GB/s": round(comb_gbs, 1)},
        },
        "roofline": {"bound": "hbm", "kernel": dom[0], "achieved": round(dom[3], 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(dom[3] / HBM_PEAK_GBS, 4),
                     "traffic": None, "bytes_per_launch": dom[1],
                     "ms_per_launch": round(float(dom[2]), 5)},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(batch, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
