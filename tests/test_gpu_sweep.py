"""Seeded random sweep of shapes and options on the GPU against the oracle.

Each case draws T, H, E, k, R, G and the routing from a fixed seed (sizes the
oracle handles in well under a second), then checks the whole path: plan
arrays and receive rows bit for bit, combine within the tolerance of
tests/gpu_util.py; with node deduplication also the staging rows and the
hierarchical combine, with load-aware forwarders the forwarder table, with
bands the banded plan.
"""

import numpy as np
import pytest
import torch

import combine_shuffling_amd as cs
import oracle
from workloads import gen

from gpu_util import DeviceRun, bits, check_combine, say, to_dev
from test_gpu_parity import hier_check

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def draw(seed):
    rng = np.random.default_rng(1000 + seed)
    E = int(rng.choice([3, 8, 17, 64, 100, 256, 1000]))
    R = int(rng.integers(1, min(E, 64) + 1))
    divisors = [g for g in range(1, R + 1) if R % g == 0]
    G = int(rng.choice(divisors))
    k = int(rng.integers(1, min(E, 16) + 1))
    T = int(rng.integers(1, 3000))
    H = int(8 * rng.integers(1, 48))
    routing = str(rng.choice(["uniform", "zipf"]))
    return T, H, E, k, R, G, routing


@pytest.mark.parametrize("seed", range(96))
def test_random_shape(seed, dev):
    T, H, E, k, R, G, routing = draw(seed)
    wl = gen.custom(T, H, E, k, R, G, routing=routing, seed=seed)
    batch = gen.make_batch(wl)
    N = R // G
    dedup = N > 1
    load_aware = dedup and seed % 2 == 1 and R * N <= 1024
    say(f"[sweep {seed}] {wl.describe()} dedup={dedup} load_aware={load_aware}")
    p = oracle.route_plan(batch.topk_idx, E, R, G, forwarders="load_aware" if load_aware else "static")
    run = DeviceRun(batch, dev, node_dedup=dedup, load_aware=load_aware).route().dispatch()
    torch.cuda.synchronize()
    plan = run.plan
    assert plan.status() == 0
    assert np.array_equal(plan.read("counts"), p["counts"])
    assert np.array_equal(plan.read("slot_of").reshape(T, k), p["slot_of"])
    assert run.guards_intact()
    recv = bits(run.recv)
    assert np.array_equal(recv, oracle.dispatch(batch.x, p))
    if dedup:
        D = p["num_staged"]
        assert np.array_equal(bits(run.staging)[:D], oracle.dedup_stage_a(batch.x, p))
        assert np.array_equal(plan.read("forwarders").reshape(R, N), p["forwarders"])
    out = run.combine(out_dtype=torch.bfloat16)
    check_combine(bits(out), recv, batch.topk_w, p["slot_of"], False, wl.name)
    if dedup:  # the hierarchical combine: partials and output
        hier_check(batch, dev, load_aware)


@pytest.mark.parametrize("seed", range(32))
def test_random_banded_pipeline(seed, dev):
    rng = np.random.default_rng(2000 + seed)
    E = int(rng.choice([8, 64, 100, 256]))
    R = int(rng.integers(1, min(E, 16) + 1))
    k = int(rng.integers(1, min(E, 8) + 1))
    T = int(rng.integers(256, 6000))
    H = int(64 * rng.integers(1, 5))
    band = int(256 * rng.integers(1, 9))
    wl = gen.custom(T, H, E, k, R, seed=seed)
    batch = gen.make_batch(wl)
    say(f"[sweep pipeline {seed}] {wl.describe()} band={band}")
    p = oracle.route_plan_banded(batch.topk_idx, E, R, band)
    plan = cs.Plan(T, H, E, k, R, band_tokens=band)
    recv, out = plan.pipeline(to_dev(batch.topk_idx, dev), to_dev(batch.x, dev),
                              to_dev(batch.topk_w, dev), out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert plan.status() == 0
    assert np.array_equal(plan.read("slot_of").reshape(T, k), p["slot_of"])
    got = bits(recv)
    assert np.array_equal(got, oracle.dispatch(batch.x, p))
    check_combine(out.cpu().numpy(), got, batch.topk_w, p["slot_of"], True, wl.name)
