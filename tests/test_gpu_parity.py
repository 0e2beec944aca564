"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bars: plan arrays, receive rows and staging rows bit-exact; combine within the
tolerance derived in tests/gpu_util.py (1e-3 relative for float32 out, one
bf16 ulp of the exact value for bf16 out, plus the float32 accumulation bound).
"""

import numpy as np
import pytest
import torch

import oracle
from workloads import gen

from gpu_util import check_combine_all, DeviceRun, bits, check_combine, check_combine_values, say, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def check_plan(run: DeviceRun, p: dict):
    wl = run.wl
    T, k = wl.num_tokens, wl.top_k
    r = run.plan
    assert r.status() == 0
    assert np.array_equal(r.read("counts"), p["counts"])
    assert np.array_equal(r.read("expert_offsets"), p["expert_offsets"])
    assert np.array_equal(r.read("rank_offsets"), p["rank_offsets"])
    assert np.array_equal(r.read("slot_of").reshape(T, k), p["slot_of"])
    assert np.array_equal(r.read("row_src"), p["row_src"])
    if run.dedup:
        D = p["num_staged"]
        assert int(r.read("num_staged")[0]) == D
        assert np.array_equal(r.read("stage_offsets"), p["stage_offsets"])
        assert np.array_equal(r.read("stage_of").reshape(T, k), p["stage_of"])
        assert np.array_equal(r.read("stage_src")[:D], p["stage_src"])
        assert np.array_equal(r.read("forwarders").reshape(wl.num_ranks, -1), p["forwarders"])


def full_check(batch, dev, dedup=None, combine_tokens=None, traffic=False, load_aware=False):
    wl = batch.workload
    say(f"[parity] {wl.describe()} dedup={dedup} load_aware={load_aware}")
    p = oracle.route_plan(batch.topk_idx, wl.num_experts, wl.num_ranks, wl.ranks_per_node,
                          forwarders="load_aware" if load_aware else "static")
    run = DeviceRun(batch, dev, node_dedup=dedup, load_aware=load_aware).route().dispatch()
    torch.cuda.synchronize()
    check_plan(run, p)
    assert run.guards_intact()
    recv = bits(run.recv)
    assert np.array_equal(recv, oracle.dispatch(batch.x, p)), "receive rows differ"
    if run.dedup:
        D = p["num_staged"]
        assert np.array_equal(bits(run.staging)[:D], oracle.dedup_stage_a(batch.x, p))
    if traffic:
        R, N = wl.num_ranks, wl.num_ranks // wl.ranks_per_node
        assert np.array_equal(run.plan.read("send_rows").reshape(R, R), p["send_rows"])
        assert np.array_equal(run.plan.read("send_copies").reshape(R, R), p["send_copies"])
        assert np.array_equal(run.plan.read("node_copies").reshape(R, N), p["node_copies"])
    for out_dtype in (torch.bfloat16, torch.float32):
        out = run.combine(out_dtype=out_dtype)
        o = out.cpu().numpy() if out_dtype == torch.float32 else bits(out)
        if combine_tokens is None:
            check_combine_all(o, recv, batch.topk_w, p["slot_of"], out_dtype == torch.float32,
                              wl.name)
        else:
            tok = combine_tokens
            check_combine(o[tok], recv, batch.topk_w[tok], p["slot_of"][tok],
                          out_dtype == torch.float32, wl.name)
    return run, p


# -- small shapes: several tiles, ragged tails, odd k / E / R / G ---------------

SMALL = [
    # T,    H,   E,  k, R, G, routing
    (1, 8, 1, 1, 1, 1, "uniform"),
    (5, 16, 3, 3, 3, 3, "uniform"),
    (255, 64, 8, 2, 2, 2, "uniform"),
    (257, 64, 8, 2, 2, 1, "uniform"),
    (1000, 40, 24, 5, 7, 7, "uniform"),
    (3001, 128, 100, 6, 7, 7, "uniform"),
    (4099, 256, 64, 8, 8, 2, "uniform"),
    (777, 72, 1024, 16, 16, 4, "uniform"),
    (2050, 24, 13, 13, 13, 13, "uniform"),
    (600, 64, 128, 8, 8, 8, "zipf"),
    (20000, 16, 30, 4, 6, 3, "uniform"),       # two 256-token passes per tile
    (40000, 8, 256, 8, 64, 8, "uniform"),     # three passes per tile
    (1500, 64, 1024, 16, 1024, 1, "uniform"),  # most experts and ranks: 1024 one-rank nodes
    (1, 64, 1024, 16, 64, 8, "uniform"),       # one token, dedup
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: "T{}-H{}-E{}-k{}-R{}-G{}".format(*c[:6]))
def test_small_shapes(case, dev):
    T, H, E, k, R, G, routing = case
    kw = dict(zipf_s=1.2) if routing == "zipf" else {}
    batch = gen.make_batch(gen.custom(T, H, E, k, R, G, routing=routing, seed=T, **kw))
    full_check(batch, dev, traffic=True)
    if R // G > 1:
        full_check(batch, dev, dedup=True)


# -- the five workloads at full size ----------------------------------------

@pytest.mark.parametrize("name", gen.WORKLOAD_ORDER)
def test_workload_full_size(name, dev):
    # every token's combine is compared (in chunks of tokens)
    full_check(gen.make_batch(gen.get(name)), dev, traffic=True)


@pytest.mark.parametrize("case", [
    # T,    H,   E,   k,  R,  G  -- staging rows past one 224 MiB chunk
    (2500, 7168, 64, 8, 16, 2),   # 2 chunks (the bound counts min(k, N) = 8 rows a token)
    (4999, 7168, 32, 8, 8, 1),    # 3 chunks of 1667 tokens, the last ragged; 8 nodes
])
def test_dedup_dispatch_in_chunks(case, dev):
    # Hop 1 and hop 2 run chunk by chunk over consecutive tokens; the rows
    # must be those of the whole-batch oracle.
    T, H, E, k, R, G = case
    full_check(gen.make_batch(gen.custom(T, H, E, k, R, G, seed=T)), dev)


def test_dedup_workload_single_hop_too(dev):
    # The DeepSeek-V3-like routing through the single-hop path gives the same rows.
    batch = gen.make_batch(gen.get("dsv3"))
    p = oracle.route_plan(batch.topk_idx, 256, 64, 8)
    run = DeviceRun(batch, dev, node_dedup=False).route().dispatch()
    torch.cuda.synchronize()
    assert np.array_equal(bits(run.recv), oracle.dispatch(batch.x, p))


# -- exact special cases of combine --------------------------------------------

def test_combine_one_hot_is_bit_exact_gather(dev):
    batch = gen.make_batch(gen.custom(3000, 256, 64, 8, 4, 4, seed=3))
    T, k = batch.topk_idx.shape
    pick = np.random.default_rng(5).integers(0, k, T)
    w = np.zeros((T, k), dtype=np.float32)
    w[np.arange(T), pick] = 1.0
    p = oracle.route_plan(batch.topk_idx, 64, 4)
    run = DeviceRun(batch, dev).route().dispatch()
    y = np.random.default_rng(6).integers(0, 0x7F00, (T * k, 256), dtype=np.uint16)
    out = run.combine(y=to_dev(y, dev), w=to_dev(w, dev))
    assert np.array_equal(bits(out), y[p["slot_of"][np.arange(T), pick]])


@pytest.mark.parametrize("k", [1, 2, 4, 8, 16])
def test_identity_roundtrip_power_of_two_exact(k, dev):
    batch = gen.make_batch(gen.custom(2000, 128, 32, k, 4, 2, seed=k))
    T = batch.topk_idx.shape[0]
    w = np.full((T, k), 1.0 / k, dtype=np.float32)
    run = DeviceRun(batch, dev).route().dispatch()
    out = run.combine(w=to_dev(w, dev))
    assert np.array_equal(bits(out), batch.x)


@pytest.mark.parametrize("name", ["tiny", "olmoe", "nondiv"])
def test_roundtrip_renormalised_within_one_ulp(name, dev):
    batch = gen.make_batch(gen.get(name))
    run = DeviceRun(batch, dev).route().dispatch()
    out = bits(run.combine())
    assert int(oracle.bf16_ulp_distance(out, batch.x).max()) <= 1


# -- behaviour ------------------------------------------------------------------

def test_deterministic_and_reusable(dev):
    batch = gen.make_batch(gen.custom(5000, 512, 100, 6, 7, 7, seed=9))
    run = DeviceRun(batch, dev).route().dispatch()
    a = bits(run.recv).copy()
    o1 = bits(run.combine())
    run.recv.fill_(-1)
    run.route().dispatch()
    assert np.array_equal(bits(run.recv), a)
    run.dispatch()           # a plan serves many dispatch / combine calls
    assert np.array_equal(bits(run.recv), a)
    assert np.array_equal(bits(run.combine()), o1)


def test_empty_batch(dev):
    import combine_shuffling_amd as cs

    idx = torch.zeros((0, 4), dtype=torch.int32, device=dev)
    plan = cs.route_plan(idx, 16, 4, 64)
    recv, _ = cs.dispatch(plan, torch.zeros((0, 64), dtype=torch.bfloat16, device=dev))
    out = cs.combine(plan, recv, torch.zeros((0, 4), dtype=torch.float32, device=dev))
    assert recv.shape == (0, 64) and out.shape == (0, 64)
    assert plan.status() == 0
    assert plan.read("counts").tolist() == [0] * 16
    assert plan.read("rank_offsets").tolist() == [0] * 5


def test_bad_routing_is_flagged_and_memory_safe(dev):
    from combine_shuffling_amd import _abi

    batch = gen.make_batch(gen.custom(1500, 64, 16, 4, 4, 2, seed=2))
    idx = batch.topk_idx.copy()
    idx[3, 1] = 16          # out of range
    idx[10, 2] = -5         # negative
    idx[700, 3] = idx[700, 0]  # repeated in a row
    batch.topk_idx = idx
    for dedup in (False, True):
        run = DeviceRun(batch, dev, node_dedup=dedup).route().dispatch()
        assert run.plan.status() == _abi.ERR_BAD_ROUTING
        assert run.guards_intact()
        so = run.plan.read("slot_of").reshape(1500, 4)
        assert so[3, 1] == -1 and so[10, 2] == -1 and so[700, 3] == -1 and so[700, 0] >= 0
        assert int(run.plan.read("counts").sum()) == 1500 * 4 - 3
        run.combine()
    # a clean routing afterwards clears the status
    good = gen.make_batch(gen.custom(1500, 64, 16, 4, 4, 2, seed=2))
    run = DeviceRun(good, dev).route()
    assert run.plan.status() == 0


def test_bad_routing_in_chunked_dedup_dispatch(dev):
    # Bad ids in both chunks of a 2-chunk deduplicated dispatch: flagged,
    # dropped slots -1, nothing written past the buffers, and the
    # hierarchical combine and the fp8 dispatch run over the same plan.
    from combine_shuffling_amd import _abi

    T, H, k = 2500, 7168, 8
    batch = gen.make_batch(gen.custom(T, H, 64, k, 16, 2, seed=4))
    idx = batch.topk_idx.copy()
    idx[5, 3] = 64             # out of range, first chunk
    idx[2000, 6] = -1          # negative, second chunk
    idx[1700, 1] = idx[1700, 0]  # repeated, second chunk
    batch.topk_idx = idx
    run = DeviceRun(batch, dev, node_dedup=True).route().dispatch()
    assert run.plan.status() == _abi.ERR_BAD_ROUTING
    assert run.guards_intact()
    so = run.plan.read("slot_of").reshape(T, k)
    assert so[5, 3] == -1 and so[2000, 6] == -1 and so[1700, 1] == -1 and so[1700, 0] >= 0
    assert int(run.plan.read("counts").sum()) == T * k - 3
    smax = run.plan.staging_rows_max
    part_full = torch.full((smax + 2, H), float("nan"), dtype=torch.float32, device=dev)
    run.plan.combine_hier(run.recv, run.w, partials=part_full[:smax])
    torch.cuda.synchronize()
    assert torch.isnan(part_full[smax:]).all(), "hop 1 wrote past the partials"
    nb = run.plan.scale_blocks
    codes_full = torch.full((run.plan.recv_rows + 2, H), 0x55, dtype=torch.uint8, device=dev)
    stage_full = torch.full((smax + 2, H), 0x55, dtype=torch.uint8, device=dev)
    run.plan.dispatch_fp8(run.x, codes_full[:run.plan.recv_rows],
                          torch.empty((run.plan.recv_rows, nb), dtype=torch.float32, device=dev),
                          stage_full[:smax], torch.empty((smax, nb), dtype=torch.float32, device=dev))
    torch.cuda.synchronize()
    assert bool((codes_full[run.plan.recv_rows:] == 0x55).all())
    assert bool((stage_full[smax:] == 0x55).all())
    assert run.plan.status() == _abi.ERR_BAD_ROUTING


def test_plan_reads_and_combine_without_dispatch(dev):
    # With no dispatch since the route, plan reads and combine finish the plan
    # themselves (one thread per token).
    batch = gen.make_batch(gen.custom(2500, 64, 40, 6, 8, 2, seed=4))
    p = oracle.route_plan(batch.topk_idx, 40, 8, 2)
    y = oracle.dispatch(batch.x, p)
    for dedup in (False, True):
        run = DeviceRun(batch, dev, node_dedup=dedup).route()
        check_plan(run, p)
        out = run.combine(y=to_dev(y, dev), out_dtype=torch.float32)
        check_combine(out.cpu().numpy(), y, batch.topk_w, p["slot_of"], True, "no-dispatch")
        # combine straight after a fresh route, no reads in between
        run.route()
        out = run.combine(y=to_dev(y, dev))
        check_combine(bits(out), y, batch.topk_w, p["slot_of"], False, "no-dispatch-bf16")


@pytest.mark.parametrize("case", [
    (2048, 64, 64, 4, 16, 4), (3001, 40, 30, 5, 6, 2), (777, 24, 1024, 16, 32, 8), (20000, 16, 64, 8, 32, 4),
    (1800, 32, 64, 16, 32, 1),    # R * N = 1024 owner-node pairs, the most the scan holds
    (4096, 16, 256, 8, 64, 4),    # 64 owners in each of 16 nodes: a full wave per node
    (1500, 32, 256, 8, 128, 16),  # more than 64 owners: ranked through the LDS tables
    (2000, 16, 192, 6, 96, 32)],
    ids=lambda c: "T{}-H{}-E{}-k{}-R{}-G{}".format(*c))
def test_load_aware_forwarders(case, dev):
    T, H, E, k, R, G = case
    batch = gen.make_batch(gen.custom(T, H, E, k, R, G, seed=T))
    full_check(batch, dev, dedup=True, load_aware=True)


def test_load_aware_forwarders_dsv3(dev):
    full_check(gen.make_batch(gen.get("dsv3")), dev, load_aware=True)


def hier_check(batch, dev, load_aware, tokens=None):
    wl = batch.workload
    say(f"[hier] {wl.describe()} load_aware={load_aware}")
    p = oracle.route_plan(batch.topk_idx, wl.num_experts, wl.num_ranks, wl.ranks_per_node,
                          forwarders="load_aware" if load_aware else "static")
    run = DeviceRun(batch, dev, node_dedup=True, load_aware=load_aware).route().dispatch()
    y = bits(run.recv)
    tok = np.arange(wl.num_tokens) if tokens is None else np.asarray(tokens)
    # The plan restricted to the checked tokens and their staging rows, renumbered.
    rows = np.unique(p["stage_of"][tok])
    sub = dict(slot_of=p["slot_of"][tok], stage_of=np.searchsorted(rows, p["stage_of"][tok]),
               stage_src=np.searchsorted(tok, p["stage_src"][rows]),
               stage_node=p["stage_node"][rows], num_staged=len(rows))
    w = batch.topk_w[tok]
    ref, ref_part = oracle.combine_hierarchical(y, w, sub)
    yv = oracle.bf16_to_f32(y).astype(np.float64)
    k, N = wl.top_k, wl.num_ranks // wl.ranks_per_node
    # a partial is an FMA chain over at most k slots
    part_scale = np.zeros_like(ref_part)
    for j in range(k):
        np.add.at(part_scale, sub["stage_of"][:, j], np.abs(w[:, j:j + 1]) * np.abs(yv[sub["slot_of"][:, j]]))
    D = p["num_staged"]
    for out_dtype in (torch.float32, torch.bfloat16):
        part = torch.full((run.plan.staging_rows_max, wl.hidden), float("nan"),
                          dtype=torch.float32, device=dev)
        out = run.plan.combine_hier(run.recv, run.w, partials=part, out_dtype=out_dtype)
        torch.cuda.synchronize()
        assert not torch.isnan(part[:D]).any(), "a staging row's partial was not written"
        gp = part[torch.as_tensor(rows, device=dev)].cpu().numpy().astype(np.float64)
        perr = np.abs(gp - ref_part)
        assert np.all(perr <= k * 2.0 ** -24 * part_scale * 1.001), float(perr.max())
        o = out.cpu().numpy() if out_dtype == torch.float32 else bits(out)
        check_combine_values(o[tok], ref, yv, w, sub["slot_of"], out_dtype == torch.float32,
                             wl.name + " hier", roundings=k + N)


@pytest.mark.parametrize("load_aware", [False, True])
@pytest.mark.parametrize("case", [
    (1000, 64, 32, 4, 8, 2), (3001, 40, 30, 5, 6, 2), (777, 24, 1024, 16, 32, 8),
    (2048, 256, 256, 8, 64, 8)], ids=lambda c: "T{}-H{}-E{}-k{}-R{}-G{}".format(*c))
def test_hierarchical_combine(case, load_aware, dev):
    T, H, E, k, R, G = case
    hier_check(gen.make_batch(gen.custom(T, H, E, k, R, G, seed=T + k)), dev, load_aware)


def test_hierarchical_combine_dsv3(dev):
    batch = gen.make_batch(gen.get("dsv3"))
    T = batch.workload.num_tokens
    tok = np.unique(np.concatenate([[0, T - 1], np.random.default_rng(9).integers(0, T, 512)]))
    hier_check(batch, dev, False, tokens=tok)


def test_hierarchical_combine_in_chunks(dev):
    # 4999 tokens of up to 8 partial rows of 7168 floats: both hops run in 3
    # chunks of consecutive tokens, the last ragged.
    batch = gen.make_batch(gen.custom(4999, 7168, 32, 8, 8, 1, seed=21))
    T = batch.workload.num_tokens
    tok = np.unique(np.concatenate([[0, 1666, 1667, 3333, 3334, T - 1],
                                    np.random.default_rng(10).integers(0, T, 256)]))
    hier_check(batch, dev, False, tokens=tok)


def test_hierarchical_combine_without_dispatch(dev):
    # Route, then combine rows that were placed by someone else: the plan fills
    # its per-slot tables itself.
    import combine_shuffling_amd as cs

    batch = gen.make_batch(gen.custom(900, 32, 64, 6, 16, 4, seed=17))
    wl = batch.workload
    p = oracle.route_plan(batch.topk_idx, wl.num_experts, wl.num_ranks, wl.ranks_per_node)
    y = oracle.dispatch(batch.x, p)
    plan = cs.Plan(wl.num_tokens, wl.hidden, wl.num_experts, wl.top_k, wl.num_ranks,
                   wl.ranks_per_node, True)
    plan.route(to_dev(batch.topk_idx, dev))
    out = plan.combine_hier(to_dev(y, dev), to_dev(batch.topk_w, dev), out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref, _ = oracle.combine_hierarchical(y, batch.topk_w, p)
    yv = oracle.bf16_to_f32(y).astype(np.float64)
    check_combine_values(out.cpu().numpy(), ref, yv, batch.topk_w, p["slot_of"], True,
                         "hier without dispatch", roundings=wl.top_k + 4)
