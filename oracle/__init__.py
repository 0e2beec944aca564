"""Plain CPU oracle for the MoE expert-parallel shuffle (route plan, dispatch,
node-deduplicated dispatch, combine).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute anything in this package: only the tests, the smoke check and the
benchmark's CPU-baseline leg use it.  It shares no code with the HIP library
(``combine_shuffling_amd``) and imports nothing from it; the two meet only in
the seeded input generator (``workloads.gen``), which holds none of the
shuffle's arithmetic.

Every result here has a plain definition (data movement plus one weighted
sum), so each function writes that definition out with numpy; floating-point
sums are taken in float64.  ``oracle.brute`` re-derives the same results with
pure-Python loops for tiny inputs.  Sources, by page title and section:

  * FUSCO article (aigc.bar, "FUSCO ... breaks the MoE communication
    bottleneck"), sections "pain points" (data shuffling under expert
    parallelism), "core innovation" (gather-send driven by segment
    descriptors, scatter-recv into the final layout) and "load balancing and
    cross-node deduplication" (one copy per destination node through a
    forwarding GPU, then intra-node fan-out);
  * INC-MoE abstract (weekinpapers 2610.36339): dispatch sends tokens to the
    ranks holding their experts, combine returns expert outputs to each
    token's owner; the AllGather / ReduceScatter formulation;
  * INC-MoE abstract: tokens partitioned into bands that pass through the
    dispatch / expert / combine pipeline one after another
    (``route_plan_banded``: each band routed as its own batch);
  * TensorRT-LLM PR #13888 ("support non-divisible EP in MoE alltoall"):
    the ceil/floor contiguous expert-to-rank partition, its printed cases,
    and the rejection of fewer experts than ranks.

Parity status: every function is pinned by tests under ``tests/`` that do not
re-run its own formula (printed values, closed forms, invariants, library
special cases, brute force); none is "parity unpinned".
"""

from .bf16 import bf16_to_f32, f32_to_bf16_rne, bf16_ulp_distance  # noqa: F401
from .partition import expert_partition, rank_of_expert, token_owners  # noqa: F401
from .shuffle import (  # noqa: F401
    RoutingError,
    validate_routing,
    expert_counts,
    route_plan,
    route_plan_banded,
    dispatch,
    dedup_stage_a,
    dedup_stage_b,
    combine,
    combine_by_rank_partials,
    combine_hierarchical,
    load_aware_forwarders,
    roundtrip,
)
