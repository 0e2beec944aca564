"""GPU parity of banded plans and of the one-launch banded pipeline.

Banded plans (each band of consecutive tokens routed as its own batch) run
through the ordinary calls must reproduce the oracle's banded plan bit for bit
(plan arrays, receive rows) and the combine within the tolerance of
tests/gpu_util.py.  The pipeline (route, dispatch and combine of every band in
one persistent launch) must give exactly what the separate calls give on the
same plan: the same kernels' arithmetic in the same order, so receive rows,
plan arrays and both output types are compared bit for bit.
"""

import dataclasses

import numpy as np
import pytest
import torch

import combine_shuffling_amd as cs
import oracle
from workloads import gen

from gpu_util import bits, check_combine, say, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def _plan(wl, band):
    return cs.Plan(wl.num_tokens, wl.hidden, wl.num_experts, wl.top_k, wl.num_ranks,
                   band_tokens=band)


def check_banded_plan(plan, p, T, k):
    nb = p["num_bands"]
    assert plan.bands == nb
    assert plan.status() == 0
    assert np.array_equal(plan.read("counts").reshape(nb, -1), p["counts"])
    assert np.array_equal(plan.read("expert_offsets").reshape(nb, -1), p["expert_offsets"])
    assert np.array_equal(plan.read("rank_offsets").reshape(nb, -1), p["rank_offsets"])
    assert np.array_equal(plan.read("slot_of").reshape(T, k), p["slot_of"])
    assert np.array_equal(plan.read("row_src"), p["row_src"])


def poisoned(rows, H, dev, dtype=torch.int16):
    full = torch.full((rows + 4, H), -1, dtype=dtype, device=dev)
    return full, full[:rows]


def run_separate(batch, band, dev, out_dtype):
    wl = batch.workload
    plan = _plan(wl, band)
    plan.route(to_dev(batch.topk_idx, dev))
    recv_full, recv = poisoned(plan.recv_rows, wl.hidden, dev)
    plan.dispatch(to_dev(batch.x, dev), recv)
    out = plan.combine(recv, to_dev(batch.topk_w, dev), out_dtype=out_dtype)
    torch.cuda.synchronize()
    assert bool((recv_full[plan.recv_rows:] == -1).all())
    return plan, recv, out


def run_pipeline(batch, band, dev, out_dtype, plan=None, repeats=1):
    wl = batch.workload
    plan = _plan(wl, band) if plan is None else plan
    recv_full, recv = poisoned(plan.recv_rows, wl.hidden, dev)
    out_full = torch.full((wl.num_tokens + 2, wl.hidden), float("nan"), dtype=out_dtype, device=dev)
    idx, x, w = to_dev(batch.topk_idx, dev), to_dev(batch.x, dev), to_dev(batch.topk_w, dev)
    for _ in range(repeats):
        plan.pipeline(idx, x, w, recv, out_full[: wl.num_tokens], out_dtype)
    torch.cuda.synchronize()
    assert bool((recv_full[plan.recv_rows:] == -1).all()), "pipeline wrote past recv"
    assert bool(torch.isnan(out_full[wl.num_tokens:].float()).all()), "pipeline wrote past out"
    return plan, recv, out_full[: wl.num_tokens]


def full_check(batch, band, dev, tokens=None):
    wl = batch.workload
    T, k = wl.num_tokens, wl.top_k
    say(f"[pipeline] {wl.describe()} band={band}")
    p = oracle.route_plan_banded(batch.topk_idx, wl.num_experts, wl.num_ranks, band)
    ref_recv = oracle.dispatch(batch.x, p)
    tok = np.arange(T) if tokens is None else tokens
    for out_dtype in (torch.bfloat16, torch.float32):
        plan_s, recv_s, out_s = run_separate(batch, band, dev, out_dtype)
        check_banded_plan(plan_s, p, T, k)
        assert np.array_equal(bits(recv_s), ref_recv), "banded receive rows differ"
        plan_p, recv_p, out_p = run_pipeline(batch, band, dev, out_dtype)
        check_banded_plan(plan_p, p, T, k)
        assert np.array_equal(bits(recv_p), ref_recv), "pipeline receive rows differ"
        if out_dtype == torch.float32:
            a, b = out_p.cpu().numpy(), out_s.cpu().numpy()
            assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), "pipeline out != separate"
            check_combine(a[tok], ref_recv, batch.topk_w[tok], p["slot_of"][tok], True, wl.name)
        else:
            a, b = bits(out_p), bits(out_s)
            assert np.array_equal(a, b), "pipeline out != separate"
            check_combine(a[tok], ref_recv, batch.topk_w[tok], p["slot_of"][tok], False, wl.name)


SMALL = [
    # T,    H,   E,   k,  R, band     (the pipeline needs H % 64 == 0)
    (1000, 64, 32, 4, 8, 256),       # ragged last band (232 tokens)
    (4096, 128, 64, 8, 4, 512),
    (3001, 192, 30, 5, 6, 768),      # 3 segments per row, the last partial; E % R != 0
    (8192, 64, 100, 6, 7, 256),      # 32 bands
    (777, 64, 1024, 16, 32, 512),    # E = 1024: two tiles per band fill the scan LDS
    (300, 256, 8, 1, 2, 256),        # k = 1
    (200, 64, 16, 4, 4, 256),        # one band (band >= T)
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: "T{}-H{}-E{}-k{}-R{}-B{}".format(*c))
def test_pipeline_small(case, dev):
    T, H, E, k, R, band = case
    full_check(gen.make_batch(gen.custom(T, H, E, k, R, R, seed=T + band)), band, dev)


def test_pipeline_olmoe(dev):
    batch = gen.make_batch(gen.get("olmoe"))
    T = batch.workload.num_tokens
    sample = np.unique(np.concatenate([[0, T - 1], np.random.default_rng(4).integers(0, T, 768)]))
    full_check(batch, 512, dev, tokens=sample)


def test_pipeline_repeated_calls_reuse_counters(dev):
    # Three launches on one workspace with different routings: each must see
    # its counters cleared by the previous launch's last block.
    plan = None
    for seed in (1, 2, 3):
        batch = gen.make_batch(gen.custom(2048, 64, 64, 8, 4, 4, seed=seed))
        wl = batch.workload
        p = oracle.route_plan_banded(batch.topk_idx, 64, 4, 256)
        plan, recv, out = run_pipeline(batch, 256, dev, torch.float32, plan=plan, repeats=2)
        assert plan.status() == 0
        assert np.array_equal(bits(recv), oracle.dispatch(batch.x, p))
        check_combine(out.cpu().numpy(), oracle.dispatch(batch.x, p), batch.topk_w, p["slot_of"],
                      True, wl.name)


def test_pipeline_on_a_workspace_holding_stale_counters(dev):
    # A caller's workspace may hold anything (a reused allocation, another
    # plan's routing): every launch zeroes its counters first, so stale
    # values cannot let a ticket pass its wait early.
    batch = gen.make_batch(gen.custom(2048, 64, 64, 8, 4, 4, seed=9))
    wl = batch.workload
    p = oracle.route_plan_banded(batch.topk_idx, 64, 4, 256)
    plan = _plan(wl, 256)
    ws = torch.full((plan.workspace_bytes,), 0x7F, dtype=torch.uint8, device=dev)
    idx, x, w = to_dev(batch.topk_idx, dev), to_dev(batch.x, dev), to_dev(batch.topk_w, dev)
    for fill in (0x7F, 0x01):
        ws.fill_(fill)          # every counter large, then every counter small
        recv, out = plan.pipeline(idx, x, w, out_dtype=torch.float32, workspace=ws)
        torch.cuda.synchronize()
        assert plan.status() == 0
        assert np.array_equal(bits(recv), oracle.dispatch(batch.x, p))
        check_combine(out.cpu().numpy(), oracle.dispatch(batch.x, p), batch.topk_w, p["slot_of"],
                      True, wl.name)


def test_pipeline_bad_routing_flagged(dev):
    batch = gen.make_batch(gen.custom(1024, 64, 16, 4, 4, 4, seed=5))
    idx = batch.topk_idx.copy()
    idx[700, 1] = 99            # out of range, in the third band
    idx[100, 2] = idx[100, 0]   # repeated, in the first band
    wl = batch.workload
    plan = _plan(wl, 256)
    recv_full, recv = poisoned(plan.recv_rows, wl.hidden, dev)
    plan.pipeline(to_dev(idx, dev), to_dev(batch.x, dev), to_dev(batch.topk_w, dev), recv)
    torch.cuda.synchronize()
    assert plan.status() == 3
    assert bool((recv_full[plan.recv_rows:] == -1).all())
    slot_of = plan.read("slot_of").reshape(1024, 4)
    assert slot_of[700, 1] == -1 and slot_of[100, 2] == -1


def test_pipeline_bad_routing_output(dev):
    """A dropped slot between kept ones (an id out of range, a repeat): the
    pipeline's combine skips it as the separate combine does, so both output
    types match the separate calls bit for bit, and every token is its kept
    slots' weighted sum (a dropped slot weighs zero)."""
    batch = gen.make_batch(gen.custom(1024, 64, 16, 4, 4, 4, seed=5))
    idx = batch.topk_idx.copy()
    idx[700, 1] = 99
    idx[100, 2] = idx[100, 0]
    bad = dataclasses.replace(batch, topk_idx=idx)
    for out_dtype in (torch.bfloat16, torch.float32):
        plan_s, recv_s, out_s = run_separate(bad, 256, dev, out_dtype)
        plan_p, recv_p, out_p = run_pipeline(bad, 256, dev, out_dtype)
        assert plan_s.status() == 3 and plan_p.status() == 3
        slot_of = plan_p.read("slot_of").reshape(1024, 4)
        assert np.array_equal(slot_of, plan_s.read("slot_of").reshape(1024, 4))
        assert sorted(map(tuple, np.argwhere(slot_of < 0))) == [(100, 2), (700, 1)]
        y = bits(recv_p)
        assert np.array_equal(y, bits(recv_s))
        f32 = out_dtype == torch.float32
        a = out_p.cpu().numpy().view(np.uint32) if f32 else bits(out_p)
        b = out_s.cpu().numpy().view(np.uint32) if f32 else bits(out_s)
        assert np.array_equal(a, b), "pipeline out != separate"
        kept = slot_of >= 0
        w = np.where(kept, batch.topk_w, np.float32(0))
        check_combine(out_p.cpu().numpy() if f32 else a, y, w, np.where(kept, slot_of, 0), f32,
                      "bad routing")


def test_pipeline_empty_batch(dev):
    plan = cs.Plan(0, 64, 16, 4, 4, band_tokens=256)
    idx = torch.zeros((0, 4), dtype=torch.int32, device=dev)
    x = torch.zeros((0, 64), dtype=torch.bfloat16, device=dev)
    w = torch.zeros((0, 4), dtype=torch.float32, device=dev)
    recv, out = plan.pipeline(idx, x, w)
    torch.cuda.synchronize()
    assert recv.shape == (0, 64) and out.shape == (0, 64)
    assert plan.status() == 0
