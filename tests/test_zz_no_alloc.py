"""moe_route_plan_static: the route plan on the library's per-device static
workspace, for callers that cannot allocate device memory.

Checked through the C ABI against moe_route_plan with a caller workspace on
the same inputs: plan items, receive (and staging) rows and both combine
outputs bit for bit, on two calls in a row whose second batch is smaller (the
static workspace keeps the first call's contents), single hop and node
deduplicated.  The size limit is checked on the host.
"""

import ctypes

import numpy as np
import pytest
import torch

import combine_shuffling_amd as cs
from combine_shuffling_amd import _abi
from workloads import gen

from gpu_util import bits, say, to_dev


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def route_static(plan, idx, dev):
    """moe_route_plan_static, called through the C ABI."""
    stream = torch.cuda.current_stream(dev)
    st = _abi.lib().moe_route_plan_static(plan._h, ctypes.c_void_p(idx.data_ptr()),
                                          ctypes.c_void_p(stream.cuda_stream))
    assert st == _abi.OK, _abi.status_str(st)
    plan.workspace, plan.topk_idx, plan.device = None, idx, dev


ITEMS = ("status", "counts", "expert_offsets", "rank_offsets", "slot_of", "row_src")
DEDUP_ITEMS = ("num_staged", "stage_offsets", "stage_of", "stage_src", "forwarders")


def run(batch, dev, static):
    wl = batch.workload
    plan = cs.Plan(wl.num_tokens, wl.hidden, wl.num_experts, wl.top_k, wl.num_ranks,
                   wl.ranks_per_node, wl.node_dedup)
    idx, x, w = to_dev(batch.topk_idx, dev), to_dev(batch.x, dev), to_dev(batch.topk_w, dev)
    if static:
        route_static(plan, idx, dev)
    else:
        plan.route(idx)
    recv, staging = plan.dispatch(x)
    out32 = plan.combine(recv, w, out_dtype=torch.float32)
    out16 = plan.combine(recv, w)
    torch.cuda.synchronize()
    got = {k: plan.read(k) for k in ITEMS + (DEDUP_ITEMS if wl.node_dedup else ())}
    got["recv"] = bits(recv)
    if wl.node_dedup:
        D = int(got["num_staged"][0])
        got["stage_src"] = got["stage_src"][:D]   # only the first D entries are defined
        got["staging"] = bits(staging)[:D]
    got["out32"] = out32.cpu().numpy().view(np.uint32)
    got["out16"] = bits(out16)
    return got


def same(a, b, what):
    assert a.keys() == b.keys()
    for k in a:
        assert np.array_equal(a[k], b[k]), f"{what}: {k} differs"


@pytest.mark.gpu
@pytest.mark.parametrize("dedup", [False, True], ids=["single_hop", "dedup"])
def test_static_workspace_matches_caller_workspace(dedup, dev):
    # Two calls in a row, the second batch smaller than the first.
    for T, H, E, k, R, G in ((4000, 512, 64, 8, 16, 4), (700, 256, 30, 4, 8, 2)):
        batch = gen.make_batch(gen.custom(T, H, E, k, R, G if dedup else R, seed=T + H))
        say(f"[no-alloc] {batch.workload.describe()}")
        same(run(batch, dev, static=False), run(batch, dev, static=True), batch.workload.name)


@pytest.mark.gpu
def test_static_workspace_full_size_then_smaller(dev):
    # The DeepSeek-V3-like batch (node deduplication, 4.6 MB of plan), then
    # the smaller OLMoE-like one on the same static workspace.
    for name in ("dsv3", "olmoe"):
        batch = gen.make_batch(gen.get(name))
        say(f"[no-alloc] {batch.workload.describe()}")
        same(run(batch, dev, static=False), run(batch, dev, static=True), name)


def test_static_workspace_limit_is_checked_on_the_host():
    # A plan whose workspace exceeds the static buffer is refused before any
    # HIP call (this runs without a GPU).
    plan = cs.Plan(1 << 21, 64, 64, 8, 4)
    assert plan.workspace_bytes > _abi.STATIC_WORKSPACE_BYTES
    st = _abi.lib().moe_route_plan_static(plan._h, ctypes.c_void_p(0), ctypes.c_void_p(0))
    assert st == _abi.ERR_STATIC_WORKSPACE
    assert "static" in _abi.status_str(st)
    small = cs.Plan(4096, 2048, 64, 8, 4)
    assert small.workspace_bytes <= _abi.STATIC_WORKSPACE_BYTES
    assert _abi.lib().moe_route_plan_static(None, None, None) == _abi.ERR_INVALID_ARGUMENT
