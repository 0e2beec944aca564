"""Pins for the oracle's route plan, dispatch, deduplicated dispatch and combine (CPU).

Checks against things other than the oracle's own formulas: a hand-worked
example, pure-Python brute force on tiny inputs, invariants the method must
keep (counts sum to T*k, every receive row written once, each (token, node)
staged once, fan-out equal to single-hop), closed forms (round-robin
routing), and exact special cases of the combine (one-hot weights; identity
expert with power-of-two weights; per-rank partial sums).
"""

import json
import os

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st, HealthCheck

import oracle
from oracle import brute
from workloads import gen


def _plan_lists(p):
    return {k: (v.tolist() if isinstance(v, np.ndarray) else v) for k, v in p.items()}


# ---------------------------------------------------------------- hand example

def test_hand_example(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "hand_example.json")))
    idx = np.array(g["topk_idx"], dtype=np.int32)
    w = np.array(g["topk_w"], dtype=np.float32)
    p = oracle.route_plan(idx, g["E"], g["R"], g["G"])
    exp = g["expected"]
    for key in ("lo", "counts", "expert_offsets", "rank_offsets", "row_src", "slot_of", "owner",
                "send_rows", "send_copies", "node_copies", "stage_src", "stage_node",
                "stage_offsets", "stage_of"):
        assert np.asarray(p[key]).tolist() == exp[key], key
    assert p["num_staged"] == exp["num_staged"]
    # y[r] = r + 1 in every column, as bf16 (small integers are exact).
    H = 8
    y = oracle.f32_to_bf16_rne(np.repeat(np.arange(1, 9, dtype=np.float32)[:, None], H, axis=1))
    out = oracle.combine(y, w, p)
    np.testing.assert_array_equal(out[:, 0], exp["combine_row_plus_one"])
    assert np.all(out == out[:, :1])


# ------------------------------------------------------------- brute force

@st.composite
def tiny_cases(draw):
    E = draw(st.integers(1, 12))
    R = draw(st.integers(1, E))
    divisors = [g for g in range(1, R + 1) if R % g == 0]
    G = draw(st.sampled_from(divisors))
    k = draw(st.integers(1, min(E, 5)))
    T = draw(st.integers(0, 16))
    H = draw(st.sampled_from([8, 16]))
    seed = draw(st.integers(0, 2 ** 31 - 1))
    rng = np.random.default_rng(seed)
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32) if T else \
        np.zeros((0, k), dtype=np.int32)
    x = rng.integers(0, 1 << 16, (T, H), dtype=np.uint16)
    x = np.where(np.isnan(oracle.bf16_to_f32(x)), np.uint16(0x3F80), x)   # finite payload
    w = rng.standard_normal((T, k)).astype(np.float32)
    return E, R, G, k, T, H, idx, x, w


@given(tiny_cases(), st.sampled_from(["static", "load_aware"]))
@settings(max_examples=300, deadline=None, suppress_health_check=[HealthCheck.too_slow])
def test_plan_dispatch_combine_vs_brute(case, fwd_rule):
    E, R, G, k, T, H, idx, x, w = case
    p = oracle.route_plan(idx, E, R, G, forwarders=fwd_rule)
    b = brute.plan(idx.tolist(), E, R, G, forwarders=fwd_rule)
    assert p["forwarders"].tolist() == b["forwarders"]
    for key in ("counts", "expert_offsets", "rank_offsets", "row_src", "send_rows",
                "send_copies", "node_copies", "stage_src", "stage_node", "stage_offsets",
                "num_staged"):
        assert _plan_lists(p)[key] == b[key], key
    assert p["slot_of"].tolist() == b["slot_of"]
    assert p["stage_of"].tolist() == b["stage_of"]
    recv = oracle.dispatch(x, p)
    assert recv.tolist() == brute.dispatch(x.tolist(), b)
    # Deduplicated path reproduces the same receive buffer.
    staging = oracle.dedup_stage_a(x, p)
    assert np.array_equal(oracle.dedup_stage_b(staging, p), recv)
    out = oracle.combine(recv, w, p)
    ref = brute.combine(recv.tolist(), w.tolist(), b)
    assert np.array_equal(out, np.array(ref, dtype=np.float64).reshape(T, H), equal_nan=True)


# ------------------------------------------------------------- invariants

def check_plan_invariants(idx, p):
    T, k = idx.shape
    E, R, G, N = p["E"], p["R"], p["G"], p["N"]
    assert p["counts"].sum() == T * k
    assert p["expert_offsets"][-1] == T * k and np.all(np.diff(p["expert_offsets"]) >= 0)
    assert p["rank_offsets"][0] == 0 and p["rank_offsets"][-1] == T * k
    # rank d's rows are the sum of its experts' counts
    for d in range(R):
        assert p["rank_offsets"][d + 1] - p["rank_offsets"][d] == \
            p["counts"][p["lo"][d]:p["lo"][d + 1]].sum()
    # slot_of is a permutation of the receive rows and row_src its inverse
    s = p["slot_of"].ravel()
    assert np.array_equal(np.sort(s), np.arange(T * k))
    assert np.array_equal(p["row_src"][s], np.repeat(np.arange(T), k))
    # each row sits in its expert's segment; tokens ascend inside a segment
    row_expert = np.searchsorted(p["expert_offsets"], np.arange(T * k), side="right") - 1
    assert np.array_equal(row_expert[s], idx.ravel())
    seg_start = p["expert_offsets"][row_expert]
    inner = np.arange(T * k) > seg_start
    assert np.all(np.diff(p["row_src"])[inner[1:]] > 0)
    # link traffic model
    owner = p["owner"]
    per_owner = np.bincount(owner, minlength=R) * k
    assert np.array_equal(p["send_rows"].sum(axis=1), per_owner)
    assert np.all(p["send_copies"] <= p["send_rows"])
    agg = p["send_copies"].reshape(R, N, G).sum(axis=2)
    assert np.all(p["node_copies"] <= agg)
    # deduplication: each (token, node) pair staged exactly once
    D = p["num_staged"]
    pairs = set(zip(p["stage_src"].tolist(), p["stage_node"].tolist()))
    assert len(pairs) == D
    node_of_slot = p["rank_of"][idx] // G
    distinct = np.array([len(set(r)) for r in node_of_slot.tolist()]) if T else np.zeros(0)
    assert D == int(distinct.sum())
    assert T <= D <= min(k, N) * T or T == 0
    assert D == p["node_copies"].sum()
    # forwarder of each staged row is on the row's node and matches the owner's local index
    for f in range(R):
        a, b = p["stage_offsets"][f], p["stage_offsets"][f + 1]
        assert np.all(p["stage_node"][a:b] == f // G)
        assert np.all(p["forwarders"][owner[p["stage_src"][a:b]], f // G] == f)
        assert np.all(np.diff(p["stage_src"][a:b]) > 0)
    st_ = p["stage_of"]
    assert np.array_equal(p["stage_src"][st_], np.repeat(np.arange(T), k).reshape(T, k))
    assert np.array_equal(p["stage_node"][st_], node_of_slot)


@pytest.mark.parametrize("name", gen.WORKLOAD_ORDER)
def test_workload_plan_invariants(name):
    wl = gen.get(name)
    b = gen.make_batch(wl)
    p = oracle.route_plan(b.topk_idx, wl.num_experts, wl.num_ranks, wl.ranks_per_node)
    check_plan_invariants(b.topk_idx.astype(np.int64), p)
    if name == "dsv3":
        # node-limited routing: every token reaches at most 4 of 8 nodes
        nodes = p["rank_of"][b.topk_idx] // wl.ranks_per_node
        assert max(len(set(r)) for r in nodes.tolist()) <= 4
        assert p["num_staged"] <= 4 * wl.num_tokens


def test_round_robin_counts_closed_form():
    # idx[t, j] = (t*k + j) mod E gives exactly T*k/E rows per expert when E | T*k.
    for T, k, E in [(64, 2, 8), (96, 3, 12), (4096, 8, 64), (100, 6, 100)]:
        idx = ((np.arange(T)[:, None] * k + np.arange(k)[None, :]) % E).astype(np.int32)
        c = oracle.expert_counts(idx, E)
        assert np.all(c == T * k // E)


def test_single_node_dedup_is_one_copy_per_token():
    rng = np.random.default_rng(3)
    T, E, k, R, G = 300, 32, 4, 8, 4
    # every token's experts inside one node (node 0 or 1, 16 experts each)
    node = rng.integers(0, 2, T)
    idx = np.stack([node[t] * 16 + rng.permutation(16)[:k] for t in range(T)]).astype(np.int32)
    p = oracle.route_plan(idx, E, R, G)
    assert p["num_staged"] == T


@pytest.mark.parametrize("bad", [[[0, 0]], [[0, 8]], [[-1, 2]]])
def test_routing_rejected(bad):
    with pytest.raises(oracle.RoutingError):
        oracle.route_plan(np.array(bad, dtype=np.int32), 8, 2)


def test_poisoned_dispatch_writes_every_row():
    wl = gen.custom(1000, 64, 24, 5, 7, 7, seed=5)
    b = gen.make_batch(wl)
    p = oracle.route_plan(b.topk_idx, wl.num_experts, wl.num_ranks)
    recv = np.full((wl.num_tokens * wl.top_k, wl.hidden), 0xFFFF, dtype=np.uint16)
    recv[:] = oracle.dispatch(b.x, p)
    assert not np.any(np.all(recv == 0xFFFF, axis=1))
    for r in range(0, recv.shape[0], 37):
        assert np.array_equal(recv[r], b.x[p["row_src"][r]])


# ------------------------------------------------------------- combine special cases

def _abs_scale(y, w, p):
    # sum_j |w[t, j]| * |y[slot_of[t, j]]|: the size of the terms being added
    ya = np.abs(oracle.bf16_to_f32(y).astype(np.float64))
    wa = np.abs(np.asarray(w, dtype=np.float64))
    so = p["slot_of"]
    return sum(wa[:, j:j + 1] * ya[so[:, j]] for j in range(so.shape[1]))


def _case(T=512, H=64, E=16, k=4, R=4, G=2, seed=11):
    wl = gen.custom(T, H, E, k, R, G, seed=seed)
    b = gen.make_batch(wl)
    p = oracle.route_plan(b.topk_idx, E, R, G)
    return b, p


def test_combine_one_hot_is_a_gather():
    b, p = _case()
    T, k = b.topk_idx.shape
    rng = np.random.default_rng(2)
    pick = rng.integers(0, k, T)
    w = np.zeros((T, k), dtype=np.float32)
    w[np.arange(T), pick] = 1.0
    y = np.random.default_rng(4).integers(0, 0x7F00, (T * k, b.x.shape[1]), dtype=np.uint16)
    out = oracle.combine(y, w, p)
    want = oracle.bf16_to_f32(y[p["slot_of"][np.arange(T), pick]]).astype(np.float64)
    assert np.array_equal(out, want)


@pytest.mark.parametrize("k", [1, 2, 4, 8])
def test_identity_expert_power_of_two_weights_roundtrip_exact(k):
    b, p = _case(k=k, E=16)
    T = b.topk_idx.shape[0]
    w = np.full((T, k), 1.0 / k, dtype=np.float32)
    out = oracle.roundtrip(b.x, w, p)
    # k equal copies times 1/k is exact; rounding back to bf16 gives x bit for bit
    assert np.array_equal(oracle.f32_to_bf16_rne(out.astype(np.float32)), b.x)


def test_roundtrip_renormalised_weights_within_one_ulp():
    b, p = _case(k=6, E=24, R=5, G=5)
    out = oracle.roundtrip(b.x, b.topk_w, p)
    got = oracle.f32_to_bf16_rne(out.astype(np.float32))
    worst = int(oracle.bf16_ulp_distance(got, b.x).max())
    assert worst <= 1, worst


def test_combine_equals_sum_of_rank_partials():
    b, p = _case(T=700, E=20, k=5, R=6, G=3)
    y = oracle.dispatch(b.x, p)
    a = oracle.combine(y, b.topk_w, p)
    c = oracle.combine_by_rank_partials(y, b.topk_w, p)
    scale = _abs_scale(y, b.topk_w, p)
    k = b.topk_idx.shape[1]
    assert np.all(np.abs(a - c) <= 2 * k * 2.0 ** -53 * scale)


def test_combine_linear_in_weights():
    b, p = _case(T=300)
    y = oracle.dispatch(b.x, p)
    w1 = b.topk_w
    w2 = np.random.default_rng(9).standard_normal(w1.shape).astype(np.float32)
    lhs = oracle.combine(y, w1, p) + oracle.combine(y, w2, p)
    rhs = oracle.combine(y, (w1.astype(np.float64) + w2).astype(np.float32), p)
    # w1 + w2 rounds once to float32; allow that rounding on top of float64 sums
    mag = _abs_scale(y, np.abs(w1) + np.abs(w2), p)
    k = b.topk_idx.shape[1]
    assert np.all(np.abs(lhs - rhs) <= (2.0 ** -24 + 4 * k * 2.0 ** -53) * mag)


# ------------------------------------------------------------- load-aware forwarders

def test_load_aware_hand_example():
    # Node 0 loads (worked by hand): s0=5, s1=1, s2=3, s3=3 with G=2.  Ranked by
    # load, ties to the lower source: s0, s2, s3, s1; snake deal 0,1,1,0 gives
    # forwarder loads 5+1=6 and 3+3=6.
    loads = np.array([[5], [1], [3], [3]])
    fwd = oracle.shuffle.load_aware_forwarders(loads, 2)
    assert fwd[:, 0].tolist() == [0, 0, 1, 1]
    # the static rule would give (s % 2): loads 5+3=8 and 1+3=4
    per = np.bincount(fwd[:, 0], weights=loads[:, 0], minlength=2)
    assert per.tolist() == [6, 6]


def _skewed_routing(T=2048, R=16, G=4, E=64, k=4, seed=0):
    # Each quarter of the token range prefers one node: sources' loads per node
    # differ a lot, which the static same-local-index rule cannot see.
    rng = np.random.default_rng(seed)
    N = R // G
    per_node = E // N
    band = np.arange(T) * 4 // T
    idx = np.empty((T, k), dtype=np.int32)
    for t in range(T):
        fav = int(band[t]) % N
        heavy = rng.random() < 0.8
        pool = np.arange(fav * per_node, (fav + 1) * per_node) if heavy else np.arange(E)
        idx[t] = rng.permutation(pool)[:k]
    return idx, E, R, G


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_load_aware_balances_forwarders(seed):
    idx, E, R, G = _skewed_routing(seed=seed)
    st_ = oracle.route_plan(idx, E, R, G, forwarders="static")
    la = oracle.route_plan(idx, E, R, G, forwarders="load_aware")
    check_plan_invariants(idx.astype(np.int64), la)
    # same pairs staged either way, only their forwarders differ
    assert la["num_staged"] == st_["num_staged"]
    assert np.array_equal(la["node_copies"], st_["node_copies"])
    loads = lambda p: np.diff(p["stage_offsets"]).reshape(R // G, G)
    l_la, l_st = loads(la), loads(st_)
    # per node: the snake deal keeps forwarders within one source's load of each other
    biggest = la["node_copies"].max(axis=0)
    assert np.all(l_la.max(axis=1) - l_la.min(axis=1) <= biggest)
    assert l_la.max() <= l_st.max()
    # each forwarder sits on its node, and every source sends a node's copies to one forwarder
    assert np.all(la["forwarders"] // G == np.arange(R // G)[None, :])


# ------------------------------------------------------------- hierarchical combine

@given(tiny_cases(), st.sampled_from(["static", "load_aware"]))
@settings(max_examples=150, deadline=None, suppress_health_check=[HealthCheck.too_slow])
def test_hierarchical_combine_vs_brute(case, fwd_rule):
    E, R, G, k, T, H, idx, x, w = case
    p = oracle.route_plan(idx, E, R, G, forwarders=fwd_rule)
    b = brute.plan(idx.tolist(), E, R, G, forwarders=fwd_rule)
    y = oracle.dispatch(x, p)
    out, part = oracle.combine_hierarchical(y, w, p)
    ref = brute.combine_hierarchical(y.tolist(), w.tolist(), b)
    assert np.array_equal(out, np.array(ref, dtype=np.float64).reshape(T, H), equal_nan=True)
    assert part.shape == (p["num_staged"], H)


def test_hierarchical_combine_equals_direct():
    b = gen.make_batch(gen.custom(700, 64, 256, 8, 64, 8, routing="node_limited",
                                  nodes_per_token=4, node_score_topn=2, seed=3))
    p = oracle.route_plan(b.topk_idx, 256, 64, 8)
    y = oracle.dispatch(b.x, p)
    h, part = oracle.combine_hierarchical(y, b.topk_w, p)
    d = oracle.combine(y, b.topk_w, p)
    k, N = 8, 8
    assert np.all(np.abs(h - d) <= (k + N) * 2.0 ** -53 * 2 * _abs_scale(y, b.topk_w, p))
    # partials of one token add up, node by node, to the token's output
    t = 5
    rows = [q for q in range(p["num_staged"]) if p["stage_src"][q] == t]
    assert len(rows) == len(set(p["stage_node"][rows]))
    assert np.allclose(part[rows].sum(axis=0), d[t], rtol=0, atol=1e-12)


# ------------------------------------------------------------- banded route plan

def test_banded_hand_example(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "banded_example.json")))
    idx = np.array(g["topk_idx"], dtype=np.int32)
    p = oracle.route_plan_banded(idx, g["E"], g["R"], g["band"])
    for key in ("slot_of", "row_src", "counts", "expert_offsets", "rank_offsets"):
        assert np.asarray(p[key]).tolist() == g["expected"][key], key
    assert oracle.route_plan(idx, g["E"], g["R"])["slot_of"].tolist() == \
        g["expected"]["unbanded_slot_of"]


@given(tiny_cases(), st.integers(1, 7))
@settings(max_examples=150, deadline=None, suppress_health_check=[HealthCheck.too_slow])
def test_banded_plan_vs_brute(case, band):
    E, R, G, k, T, H, idx, x, w = case
    p = oracle.route_plan_banded(idx, E, R, band)
    b = brute.plan_banded(idx.tolist(), E, R, band)
    assert p["num_bands"] == b["num_bands"]
    for key in ("slot_of", "row_src", "counts", "expert_offsets", "rank_offsets"):
        assert np.asarray(p[key]).tolist() == b[key], key


@pytest.mark.parametrize("band", [256, 1000, 4096, 5000])
def test_banded_plan_invariants(band):
    batch = gen.make_batch(gen.custom(4096, 16, 64, 8, 4, 4, seed=2))
    idx, w = batch.topk_idx, batch.topk_w
    T, k = idx.shape
    p = oracle.route_plan_banded(idx, 64, 4, band)
    whole = oracle.route_plan(idx, 64, 4)
    if band >= T:       # one band is the unbanded plan
        for key in ("slot_of", "row_src", "counts", "expert_offsets", "rank_offsets"):
            assert np.array_equal(np.asarray(p[key]).reshape(np.asarray(whole[key]).shape), whole[key])
    assert np.array_equal(np.sort(p["slot_of"].ravel()), np.arange(T * k))
    assert np.array_equal(p["row_src"][p["slot_of"]], np.repeat(np.arange(T), k).reshape(T, k))
    assert np.array_equal(p["counts"].sum(axis=0), oracle.expert_counts(idx, 64))
    for b in range(p["num_bands"]):
        t0, t1 = b * band, min((b + 1) * band, T)
        rows = p["slot_of"][t0:t1]
        assert rows.min() >= t0 * k and rows.max() < t1 * k
        # inside a band: experts ascending, tokens ascending inside an expert
        e_of_row = np.empty(T * k, dtype=np.int64)
        e_of_row[p["slot_of"].ravel()] = idx.ravel()
        seg = slice(t0 * k, t1 * k)
        key = e_of_row[seg] * T + p["row_src"][seg]
        assert np.all(np.diff(key) > 0)
        assert p["expert_offsets"][b][0] == t0 * k and p["expert_offsets"][b][-1] == t1 * k
    # the combine of a token does not depend on where its rows sit
    y = oracle.dispatch(batch.x, p)
    assert np.array_equal(oracle.combine(y, w, p), oracle.combine(oracle.dispatch(batch.x, whole), w, whole))
    assert np.array_equal(p["send_rows"], whole["send_rows"])
