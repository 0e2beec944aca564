"""Seeded synthetic inputs for the MoE expert-parallel shuffle.

Both sides of every parity check draw their inputs from here: the CPU oracle
(under ``oracle/``) and the HIP library (``combine_shuffling_amd``).  This
module holds no shuffle arithmetic on purpose: it only draws activations and
a router's top-k choice.  It never computes an expert-to-rank partition,
counts, offsets, slot positions, staging rows or a combine.  Where a workload
needs per-rank expert ranges (the rank-local routing of the non-divisible
workload) it takes the range sizes that the workload description lists.

What the router does (not part of the shuffle, only its input):
  * gate logits ~ N(0, 1) in float32, plus a per-expert bias where the
    workload has a popularity skew;
  * top-k = the k largest logits, ties going to the lower expert id, stored
    in descending-logit order;
  * combine weights = softmax over the k selected logits (the renormalised
    top-k softmax), computed in float64 and stored as float32.

Activations are N(0, 1) float32 draws rounded to bfloat16 by torch's CPU
cast, returned as their raw uint16 bit patterns.

Random draws use ``numpy.random.default_rng(seed)``; the draw order is
activations, then logits, then the workload's own extra draws.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np


@dataclass(frozen=True)
class Workload:
    """One shuffle workload: sizes plus the router recipe that feeds it."""

    name: str
    num_tokens: int          # T
    hidden: int              # H (bf16 elements per row)
    num_experts: int         # E
    top_k: int               # k
    num_ranks: int           # R (virtual expert-parallel ranks)
    ranks_per_node: int      # G (R // G virtual nodes)
    routing: str = "uniform"  # uniform | zipf | node_limited | rank_local
    seed: int = 0
    zipf_s: float = 0.0
    nodes_per_token: int = 0          # node_limited: nodes kept per token
    node_score_topn: int = 0          # node_limited: logits summed per node
    rank_sizes: tuple = field(default=())  # rank_local: experts per rank
    p_local: float = 0.0              # rank_local: chance of one-rank routing

    @property
    def num_nodes(self) -> int:
        return self.num_ranks // self.ranks_per_node

    @property
    def node_dedup(self) -> bool:
        return self.num_nodes > 1

    def describe(self) -> str:
        return (f"{self.name}: T={self.num_tokens} H={self.hidden} "
                f"E={self.num_experts} k={self.top_k} R={self.num_ranks} "
                f"G={self.ranks_per_node} routing={self.routing} seed={self.seed}")


# The five workloads.  Each line restates the workload's own description.
WORKLOADS = {
    # Tiny shuffle: T=128, H=256, E=8, top-2 from N(0,1) gate logits, two
    # virtual ranks of four experts each, seed 0.
    "tiny": Workload("tiny-T128-H256-E8-k2-R2", 128, 256, 8, 2, 2, 2),
    # OLMoE-like prefill: T=4096, H=2048, E=64, top-8, N(0,1) logits
    # (near-uniform load), four virtual ranks of 16 experts.
    "olmoe": Workload("olmoe-prefill-T4096-H2048-E64-k8-R4", 4096, 2048, 64, 8, 4, 4),
    # Qwen3-235B-like imbalanced: T=8192, H=4096, E=128, top-8, logit bias =
    # log of a Zipf(s=1.2) mass over expert ids, eight ranks of 16 experts.
    "qwen3": Workload("qwen3-zipf1.2-T8192-H4096-E128-k8-R8", 8192, 4096, 128, 8, 8, 8,
                      routing="zipf", zipf_s=1.2),
    # DeepSeek-V3-like multi-node: T=16384, H=7168, E=256, top-8 under
    # node-limited routing (at most 4 of 8 virtual nodes per token), 64
    # virtual ranks grouped 8 per node, 4 experts per rank.
    "dsv3": Workload("dsv3-dedup-T16384-H7168-E256-k8-R64-G8", 16384, 7168, 256, 8, 64, 8,
                     routing="node_limited", nodes_per_token=4, node_score_topn=2),
    # Non-divisible EP: T=32768, H=2048, E=100 over 7 ranks holding
    # 15,15,14,14,14,14,14 experts, top-6; with probability 0.7 all of a
    # token's experts fall in one rank's range, otherwise unrestricted.
    "nondiv": Workload("nondiv-T32768-H2048-E100-k6-R7", 32768, 2048, 100, 6, 7, 7,
                       routing="rank_local", rank_sizes=(15, 15, 14, 14, 14, 14, 14),
                       p_local=0.7),
}

# Order in which the workloads are listed in the workload table.
WORKLOAD_ORDER = ("tiny", "olmoe", "qwen3", "dsv3", "nondiv")


@dataclass
class Batch:
    """Inputs of one shuffle call, all host-side numpy arrays."""

    workload: Workload
    x: np.ndarray        # [T, H] uint16 bf16 bit patterns
    topk_idx: np.ndarray  # [T, k] int32 expert ids
    topk_w: np.ndarray    # [T, k] float32 combine weights


def bf16_bits_from_f32(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 with torch's CPU cast; return uint16 bits."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def _topk_desc(logits: np.ndarray, k: int) -> np.ndarray:
    """Indices of the k largest entries per row; ties go to the lower index."""
    order = np.argsort(-logits, axis=1, kind="stable")
    return np.ascontiguousarray(order[:, :k]).astype(np.int32)


def _softmax_selected(logits: np.ndarray, idx: np.ndarray) -> np.ndarray:
    sel = np.take_along_axis(logits.astype(np.float64), idx.astype(np.int64), axis=1)
    sel = sel - sel.max(axis=1, keepdims=True)
    ex = np.exp(sel)
    return (ex / ex.sum(axis=1, keepdims=True)).astype(np.float32)


def route(wl: Workload, logits: np.ndarray, rng: np.random.Generator) -> np.ndarray:
    """The router's top-k choice for one workload (see the module docstring)."""
    T, E, k = logits.shape[0], wl.num_experts, wl.top_k
    if wl.routing in ("uniform", "zipf"):
        return _topk_desc(logits, k)
    if wl.routing == "node_limited":
        # Experts are grouped into num_nodes equal, contiguous groups (32 per
        # node for the DeepSeek-V3-like workload: 4 experts x 8 ranks).
        nn = wl.num_nodes
        per = E // nn
        grouped = logits.reshape(T, nn, per)
        top = -np.sort(-grouped, axis=2)[:, :, : wl.node_score_topn]
        score = top.sum(axis=2)                              # [T, nn]
        keep = _topk_desc(score, wl.nodes_per_token)        # [T, nodes_per_token]
        mask = np.full((T, nn), -np.inf, dtype=np.float32)
        np.put_along_axis(mask, keep.astype(np.int64), 0.0, axis=1)
        masked = logits + np.repeat(mask, per, axis=1)
        return _topk_desc(masked, k)
    if wl.routing == "rank_local":
        sizes = np.asarray(wl.rank_sizes, dtype=np.int64)
        starts = np.concatenate([[0], np.cumsum(sizes)])
        u = rng.random(T)
        r = rng.integers(0, len(sizes), T)
        out = _topk_desc(logits, k)
        local = np.nonzero(u < wl.p_local)[0]
        ids = np.arange(E)
        for rr in range(len(sizes)):
            rows = local[r[local] == rr]
            if rows.size == 0:
                continue
            inside = (ids >= starts[rr]) & (ids < starts[rr + 1])
            masked = np.where(inside[None, :], logits[rows], -np.inf).astype(np.float32)
            out[rows] = _topk_desc(masked, k)
        return out
    raise ValueError(f"unknown routing {wl.routing!r}")


def make_batch(wl: Workload, seed: int | None = None) -> Batch:
    """Draw one seeded batch for ``wl`` (activations, then logits, then extras)."""
    rng = np.random.default_rng(wl.seed if seed is None else seed)
    T, H, E = wl.num_tokens, wl.hidden, wl.num_experts
    x = bf16_bits_from_f32(rng.standard_normal((T, H), dtype=np.float32))
    logits = rng.standard_normal((T, E), dtype=np.float32)
    if wl.routing == "zipf":
        p = (np.arange(E, dtype=np.float64) + 1.0) ** (-wl.zipf_s)
        logits = (logits + np.log(p / p.sum())).astype(np.float32)
    idx = route(wl, logits, rng)
    w = _softmax_selected(logits, idx)
    return Batch(wl, x, idx, w)


def get(name: str) -> Workload:
    return WORKLOADS[name]


def custom(T: int, H: int, E: int, k: int, R: int, G: int | None = None, *,
           routing: str = "uniform", seed: int = 0, **kw) -> Workload:
    """A workload of arbitrary size for parity sweeps and edge cases."""
    G = R if G is None else G
    return Workload(f"custom-T{T}-H{H}-E{E}-k{k}-R{R}-G{G}-{routing}-s{seed}",
                    T, H, E, k, R, G, routing=routing, seed=seed, **kw)
