"""Per-launch kernel timing (moe_plan_timing) on the GPU: every kernel a call
launches is recorded, in launch order, with a positive duration and a start
offset that follows the launch order on one stream."""

import numpy as np
import pytest
import torch

import combine_shuffling_amd as cs
from workloads import gen

from gpu_util import to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


@pytest.mark.parametrize("dedup", [False, True], ids=["single_hop", "dedup"])
def test_every_launch_is_timed_in_order(dedup, dev):
    b = gen.make_batch(gen.custom(5000, 7168, 32, 8, 8, 1 if dedup else 8, seed=2))
    wl = b.workload
    plan = cs.Plan(wl.num_tokens, wl.hidden, wl.num_experts, wl.top_k, wl.num_ranks,
                   wl.ranks_per_node, dedup)
    plan.timing(64)
    plan.route(to_dev(b.topk_idx, dev))
    recv, _ = plan.dispatch(to_dev(b.x, dev))
    plan.combine(recv, to_dev(b.topk_w, dev))
    rec = plan.timing_read()
    names = [n for n, _, _ in rec]
    if dedup:
        # 5000 tokens of up to 8 staging rows of 14 KiB: three chunks, hop 2 of
        # a chunk sharing a launch with hop 1 of the next
        assert plan.chunk_tokens["dispatch"] == 1667
        assert names == ["route_count_kernel", "route_scan_kernel", "stage_a_kernel",
                         "stage_ab_kernel", "stage_ab_kernel", "stage_b_kernel", "combine_kernel"]
    else:
        assert names[0] == "route_count_kernel" and names[-1] == "combine_kernel"
        assert names[-2] in ("gather_kernel", "gather_scan_kernel")
    starts = np.array([st for _, st, _ in rec])
    ms = np.array([m for _, _, m in rec])
    assert starts[0] == 0.0 and np.all(ms > 0)
    # one stream: each kernel starts after the previous one has ended
    assert np.all(starts[1:] >= starts[:-1] + ms[:-1] - 1e-3)
    # the record was cleared; later launches past the capacity run untimed
    assert plan.timing_read() == []
    plan.timing(1)
    plan.combine(recv, to_dev(b.topk_w, dev))
    plan.combine(recv, to_dev(b.topk_w, dev))
    assert [n for n, _, _ in plan.timing_read()] == ["combine_kernel"]
    plan.timing(0)
    torch.cuda.synchronize()
