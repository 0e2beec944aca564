"""Two batches in flight: independent plans on two HIP streams, free-running,
staggered (each dispatch after the previous batch's dispatch) or planned
ahead (each route plan on a side stream while the previous batch moves).

A caller may keep a second batch's route plan, dispatch and combine running
on another stream while the first batch's are still running (the library
holds no state shared between plans).  Launches of the two batches are
interleaved, repeated, and each batch must still match the oracle to the
usual bars: plan arrays and receive rows bit-exact, combine within the
tolerance of tests/gpu_util.py.  The last tests run each workload at full size
in the schedule the benchmark picks for it, with the benchmark's cycling of
buffer sets (bf16 and fp8 payloads, direct and hierarchical combine).
"""

import numpy as np
import pytest
import torch

import combine_shuffling_amd as cs
import oracle
from oracle import fp8
from workloads import gen

from gpu_util import (bits, check_combine, check_combine_all, check_combine_chunks,
                      check_combine_values, say, to_dev)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


CASES = [
    # T,    H,   E,  k, R, G
    (1000, 256, 32, 4, 8, 8),     # single hop, fused scan in the gather
    (3001, 192, 30, 5, 6, 6),     # E % R != 0, ragged last segment
    (2048, 512, 64, 8, 8, 4),     # node dedup: two virtual nodes
    (8192, 128, 128, 8, 8, 8),    # separate scan launch (32 tiles x 128 experts)
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "T{}-H{}-E{}-k{}-R{}-G{}".format(*c))
def test_two_batches_in_flight(case, dev):
    T, H, E, k, R, G = case
    streams = [torch.cuda.Stream(dev) for _ in range(2)]
    runs = []
    for seed in (11, 12):
        b = gen.make_batch(gen.custom(T, H, E, k, R, G, seed=seed))
        wl = b.workload
        say(f"[streams] {wl.describe()}")
        plan = cs.Plan(T, H, E, k, R, G, wl.node_dedup)
        runs.append(dict(
            b=b, plan=plan, x=to_dev(b.x, dev), idx=to_dev(b.topk_idx, dev), w=to_dev(b.topk_w, dev),
            recv=torch.full((plan.recv_rows, H), -1, dtype=torch.int16, device=dev),
            st=(torch.full((plan.staging_rows_max, H), -1, dtype=torch.int16, device=dev)
                if wl.node_dedup else None),
            out=torch.full((T, H), float("nan"), dtype=torch.float32, device=dev)))
    torch.cuda.synchronize()
    for _ in range(3):
        for r, st in zip(runs, streams):
            r["plan"].route(r["idx"], stream=st)
        for r, st in zip(runs, streams):
            r["plan"].dispatch(r["x"], r["recv"], r["st"], stream=st)
        for r, st in zip(runs, streams):
            r["plan"].combine(r["recv"], r["w"], r["out"], torch.float32, stream=st)
    torch.cuda.synchronize()
    for r in runs:
        b, wl = r["b"], r["b"].workload
        p = oracle.route_plan(b.topk_idx, E, R, G)
        assert r["plan"].status() == 0
        assert np.array_equal(r["plan"].read("slot_of").reshape(T, k), p["slot_of"])
        assert np.array_equal(r["plan"].read("expert_offsets"), p["expert_offsets"])
        recv = bits(r["recv"])
        assert np.array_equal(recv, oracle.dispatch(b.x, p)), "receive rows differ"
        if wl.node_dedup:
            D = p["num_staged"]
            assert np.array_equal(bits(r["st"])[:D], oracle.dedup_stage_a(b.x, p))
        check_combine(r["out"].cpu().numpy(), recv, b.topk_w, p["slot_of"], True, wl.name)


@pytest.mark.parametrize("case", CASES[1:3], ids=lambda c: "T{}-H{}-E{}-k{}-R{}-G{}".format(*c))
def test_staggered_batches(case, dev):
    """Four batches on two streams, each batch's dispatch ordered after the
    previous batch's dispatch by an event (so it runs beside that batch's
    combine): every batch still matches the oracle."""
    T, H, E, k, R, G = case
    streams = [torch.cuda.Stream(dev) for _ in range(2)]
    done = [torch.cuda.Event() for _ in range(2)]
    runs = []
    for seed in (21, 22, 23, 24):
        b = gen.make_batch(gen.custom(T, H, E, k, R, G, seed=seed))
        wl = b.workload
        say(f"[staggered] {wl.describe()}")
        plan = cs.Plan(T, H, E, k, R, G, wl.node_dedup)
        runs.append(dict(
            b=b, plan=plan, x=to_dev(b.x, dev), idx=to_dev(b.topk_idx, dev), w=to_dev(b.topk_w, dev),
            recv=torch.full((plan.recv_rows, H), -1, dtype=torch.int16, device=dev),
            st=(torch.full((plan.staging_rows_max, H), -1, dtype=torch.int16, device=dev)
                if wl.node_dedup else None),
            out=torch.full((T, H), float("nan"), dtype=torch.float32, device=dev)))
    torch.cuda.synchronize()
    for i, r in enumerate(runs):
        st = streams[i % 2]
        r["plan"].route(r["idx"], stream=st)
        if i > 0:
            st.wait_event(done[(i - 1) % 2])
        r["plan"].dispatch(r["x"], r["recv"], r["st"], stream=st)
        done[i % 2].record(st)
        r["plan"].combine(r["recv"], r["w"], r["out"], torch.float32, stream=st)
    torch.cuda.synchronize()
    for r in runs:
        b, wl = r["b"], r["b"].workload
        p = oracle.route_plan(b.topk_idx, E, R, G)
        assert r["plan"].status() == 0
        recv = bits(r["recv"])
        assert np.array_equal(recv, oracle.dispatch(b.x, p)), "receive rows differ"
        if wl.node_dedup:
            D = p["num_staged"]
            assert np.array_equal(bits(r["st"])[:D], oracle.dedup_stage_a(b.x, p))
        check_combine(r["out"].cpu().numpy(), recv, b.topk_w, p["slot_of"], True, wl.name)


@pytest.mark.parametrize("case", CASES[1:3], ids=lambda c: "T{}-H{}-E{}-k{}-R{}-G{}".format(*c))
def test_plan_ahead_batches(case, dev):
    """Four batches: dispatch and combine on one stream, each batch's route
    plan on a second stream while the previous batch moves (ordered by
    events both ways): every batch still matches the oracle."""
    T, H, E, k, R, G = case
    main, side = torch.cuda.Stream(dev), torch.cuda.Stream(dev)
    routed = [torch.cuda.Event() for _ in range(2)]
    moving = torch.cuda.Event()
    runs = []
    for seed in (31, 32, 33, 34):
        b = gen.make_batch(gen.custom(T, H, E, k, R, G, seed=seed))
        wl = b.workload
        say(f"[plan ahead] {wl.describe()}")
        plan = cs.Plan(T, H, E, k, R, G, wl.node_dedup)
        runs.append(dict(
            b=b, plan=plan, x=to_dev(b.x, dev), idx=to_dev(b.topk_idx, dev), w=to_dev(b.topk_w, dev),
            recv=torch.full((plan.recv_rows, H), -1, dtype=torch.int16, device=dev),
            st=(torch.full((plan.staging_rows_max, H), -1, dtype=torch.int16, device=dev)
                if wl.node_dedup else None),
            out=torch.full((T, H), float("nan"), dtype=torch.float32, device=dev)))
    torch.cuda.synchronize()
    runs[0]["plan"].route(runs[0]["idx"], stream=side)
    routed[0].record(side)
    for i, r in enumerate(runs):
        main.wait_event(routed[i % 2])
        moving.record(main)
        r["plan"].dispatch(r["x"], r["recv"], r["st"], stream=main)
        r["plan"].combine(r["recv"], r["w"], r["out"], torch.float32, stream=main)
        if i + 1 < len(runs):
            side.wait_event(moving)
            runs[i + 1]["plan"].route(runs[i + 1]["idx"], stream=side)
            routed[(i + 1) % 2].record(side)
    torch.cuda.synchronize()
    for r in runs:
        b, wl = r["b"], r["b"].workload
        p = oracle.route_plan(b.topk_idx, E, R, G)
        assert r["plan"].status() == 0
        recv = bits(r["recv"])
        assert np.array_equal(recv, oracle.dispatch(b.x, p)), "receive rows differ"
        if wl.node_dedup:
            D = p["num_staged"]
            assert np.array_equal(bits(r["st"])[:D], oracle.dedup_stage_a(b.x, p))
        check_combine(r["out"].cpu().numpy(), recv, b.topk_w, p["slot_of"], True, wl.name)


def _dispatch(s, st):
    if "scale" in s:   # fp8 payload
        s["plan"].dispatch_fp8(s["x"], s["recv"], s["scale"], s["st"], s["sscale"], stream=st)
    else:
        s["plan"].dispatch(s["x"], s["recv"], s["st"], stream=st)


def _combine(s, st):
    if "part" in s:    # hierarchical combine through fp32 partials
        s["plan"].combine_hier(s["recv"], s["w"], s["part"], s["out"], stream=st)
    elif "scale" in s:
        s["plan"].combine_fp8(s["recv"], s["scale"], s["w"], s["out"], stream=st)
    else:
        s["plan"].combine(s["recv"], s["w"], s["out"], stream=st)


def _run_schedule(sets, schedule, steps, dev):
    """The benchmark's schedules over buffer sets cycled in order: step i
    uses set i % len(sets); "two_in_flight" and "staggered" run it on stream
    i % 2 (an even number of sets keeps each set on one stream), "plan_ahead"
    moves every step on one stream and routes the next on the other."""
    streams = [torch.cuda.Stream(dev), torch.cuda.Stream(dev)]
    done = [torch.cuda.Event(), torch.cuda.Event()]
    if schedule == "plan_ahead":
        main, side = streams
        routed = [torch.cuda.Event(), torch.cuda.Event()]
        moving = torch.cuda.Event()
        sets[0]["plan"].route(sets[0]["idx"], stream=side)
        routed[0].record(side)
        for i in range(steps):
            s = sets[i % len(sets)]
            main.wait_event(routed[i % 2])
            moving.record(main)
            _dispatch(s, main)
            _combine(s, main)
            if i + 1 < steps:
                s1 = sets[(i + 1) % len(sets)]
                side.wait_event(moving)
                s1["plan"].route(s1["idx"], stream=side)
                routed[(i + 1) % 2].record(side)
        return
    for i in range(steps):
        s, st = sets[i % len(sets)], streams[i % 2]
        s["plan"].route(s["idx"], stream=st)
        if schedule == "staggered" and i > 0:
            st.wait_event(done[(i - 1) % 2])
        _dispatch(s, st)
        done[i % 2].record(st)
        _combine(s, st)


@pytest.mark.parametrize("name,schedule,load_aware", [
    ("olmoe", "two_in_flight", False), ("qwen3", "staggered", False),
    ("nondiv", "staggered", False), ("dsv3", "plan_ahead", False), ("dsv3", "plan_ahead", True)])
def test_full_size_in_benchmark_schedule(name, schedule, load_aware, dev):
    """Each workload at full size in the schedule the benchmark's trial picks
    for it: four buffer sets holding four different batches (seeds 0-3 of the
    workload's recipe, so that rows taken from the wrong set would show),
    cycled over eight steps, bf16 output.  Every set's receive (and staging)
    rows are compared bit for bit, its combine on every token; on the
    DeepSeek-V3-like workload also with load-aware forwarders."""
    wl = gen.get(name)
    T, H, E, k, R, G = (wl.num_tokens, wl.hidden, wl.num_experts, wl.top_k, wl.num_ranks,
                        wl.ranks_per_node)
    sets = []
    for seed in range(4):
        b = gen.make_batch(wl, seed=seed)
        plan = cs.Plan(T, H, E, k, R, G, wl.node_dedup, load_aware)
        sets.append(dict(
            b=b, plan=plan, x=to_dev(b.x, dev), idx=to_dev(b.topk_idx, dev), w=to_dev(b.topk_w, dev),
            recv=torch.full((plan.recv_rows, H), -1, dtype=torch.int16, device=dev),
            st=(torch.full((plan.staging_rows_max, H), -1, dtype=torch.int16, device=dev)
                if wl.node_dedup else None),
            out=torch.full((T, H), float("nan"), dtype=torch.bfloat16, device=dev)))
    torch.cuda.synchronize()
    say(f"[full size, {schedule}] {wl.describe()} load_aware={load_aware}: 4 sets, 8 steps")
    _run_schedule(sets, schedule, 8, dev)
    torch.cuda.synchronize()
    for seed, s in enumerate(sets):
        b = s["b"]
        p = oracle.route_plan(b.topk_idx, E, R, G, forwarders="load_aware" if load_aware else "static")
        assert s["plan"].status() == 0
        if load_aware:
            assert np.array_equal(s["plan"].read("forwarders").reshape(R, -1), p["forwarders"])
        recv = bits(s["recv"])
        assert np.array_equal(recv, oracle.dispatch(b.x, p)), f"receive rows of set {seed}"
        if wl.node_dedup:
            D = p["num_staged"]
            assert np.array_equal(bits(s["st"])[:D], oracle.dedup_stage_a(b.x, p)), \
                f"staging rows of set {seed}"
        check_combine_all(bits(s["out"]), recv, b.topk_w, p["slot_of"], False,
                          f"{wl.name} set {seed}")


@pytest.mark.parametrize("name,schedule", [("qwen3", "staggered"), ("dsv3", "plan_ahead")])
def test_full_size_fp8_in_benchmark_schedule(name, schedule, dev):
    """The same with the fp8 payload (with node deduplication on the
    DeepSeek-V3-like workload): every set's codes and block scales bit for
    bit, staging ones too, its combine on every token against the
    oracle's float64 sum of the decoded rows."""
    wl = gen.get(name)
    T, H, E, k, R, G = (wl.num_tokens, wl.hidden, wl.num_experts, wl.top_k, wl.num_ranks,
                        wl.ranks_per_node)
    sets = []
    for seed in range(4):
        b = gen.make_batch(wl, seed=seed)
        plan = cs.Plan(T, H, E, k, R, G, wl.node_dedup)
        rows, smax, nb = plan.recv_rows, plan.staging_rows_max, plan.scale_blocks
        sets.append(dict(
            b=b, plan=plan, x=to_dev(b.x, dev), idx=to_dev(b.topk_idx, dev), w=to_dev(b.topk_w, dev),
            recv=torch.full((rows, H), 0x55, dtype=torch.uint8, device=dev),
            scale=torch.full((rows, nb), -1.0, dtype=torch.float32, device=dev),
            st=(torch.full((smax, H), 0x55, dtype=torch.uint8, device=dev) if wl.node_dedup else None),
            sscale=(torch.full((smax, nb), -1.0, dtype=torch.float32, device=dev)
                    if wl.node_dedup else None),
            out=torch.full((T, H), float("nan"), dtype=torch.bfloat16, device=dev)))
    torch.cuda.synchronize()
    say(f"[full size fp8, {schedule}] {wl.describe()}: 4 sets, 8 steps")
    _run_schedule(sets, schedule, 8, dev)
    torch.cuda.synchronize()
    for seed, s in enumerate(sets):
        b = s["b"]
        p = oracle.route_plan(b.topk_idx, E, R, G)
        assert s["plan"].status() == 0
        if wl.node_dedup:
            sc, se, rc, re = fp8.dedup_dispatch_fp8(b.x, p)
            D = p["num_staged"]
            assert np.array_equal(s["st"][:D].cpu().numpy(), sc), f"staging codes of set {seed}"
            assert np.array_equal(s["sscale"][:D].cpu().numpy().astype(np.float64), np.ldexp(1.0, se))
        else:
            rc, re = fp8.dispatch_fp8(b.x, p)
        assert np.array_equal(s["recv"].cpu().numpy(), rc), f"receive codes of set {seed}"
        assert np.array_equal(s["scale"].cpu().numpy().astype(np.float64), np.ldexp(1.0, re)), \
            f"receive scales of set {seed}"
        check_combine_chunks(
            bits(s["out"]), b.topk_w, p["slot_of"], False, f"{wl.name} fp8 set {seed}",
            lambda used, wc, sub: (fp8.combine_fp8(rc[used], re[used], wc, {"slot_of": sub}),
                                   fp8.dequantize_rows(rc[used], re[used])))


def test_full_size_hierarchical_combine_in_benchmark_schedule(dev):
    """The DeepSeek-V3-like workload with the hierarchical combine (an fp32
    partial per staging row, then the sum over nodes), staggered, four sets
    over eight steps: receive and staging rows bit for bit, the output on
    sampled tokens within the bound of k + N float32 roundings."""
    wl = gen.get("dsv3")
    T, H, E, k, R, G = (wl.num_tokens, wl.hidden, wl.num_experts, wl.top_k, wl.num_ranks,
                        wl.ranks_per_node)
    N = R // G
    sets = []
    for seed in range(4):
        b = gen.make_batch(wl, seed=seed)
        plan = cs.Plan(T, H, E, k, R, G, True)
        sets.append(dict(
            b=b, plan=plan, x=to_dev(b.x, dev), idx=to_dev(b.topk_idx, dev), w=to_dev(b.topk_w, dev),
            recv=torch.full((plan.recv_rows, H), -1, dtype=torch.int16, device=dev),
            st=torch.full((plan.staging_rows_max, H), -1, dtype=torch.int16, device=dev),
            part=torch.full((plan.staging_rows_max, H), float("nan"), dtype=torch.float32, device=dev),
            out=torch.full((T, H), float("nan"), dtype=torch.bfloat16, device=dev)))
    torch.cuda.synchronize()
    say(f"[full size hierarchical combine, staggered] {wl.describe()}: 4 sets, 8 steps")
    _run_schedule(sets, "staggered", 8, dev)
    torch.cuda.synchronize()
    rng = np.random.default_rng(8)
    tok = np.unique(np.concatenate([[0, T - 1], rng.integers(0, T, 768)]))
    for seed, s in enumerate(sets):
        b = s["b"]
        p = oracle.route_plan(b.topk_idx, E, R, G)
        assert s["plan"].status() == 0
        recv = bits(s["recv"])
        assert np.array_equal(recv, oracle.dispatch(b.x, p)), f"receive rows of set {seed}"
        D = p["num_staged"]
        assert np.array_equal(bits(s["st"])[:D], oracle.dedup_stage_a(b.x, p)), \
            f"staging rows of set {seed}"
        so = p["slot_of"][tok]
        used = np.unique(so)
        sub = np.searchsorted(used, so)
        ref = oracle.combine(recv[used], b.topk_w[tok], {"slot_of": sub})
        yv = oracle.bf16_to_f32(recv[used]).astype(np.float64)
        check_combine_values(bits(s["out"])[tok], ref, yv, b.topk_w[tok], sub, False,
                             f"{wl.name} hierarchical set {seed}", roundings=k + N)
