"""Route plan, dispatch, node-deduplicated dispatch and combine, written as
their plain definitions (oracle, test infrastructure only).

Notation: T tokens, H hidden (bf16 elements per row), E experts, k experts
per token, R ranks, G ranks per node, N = R // G nodes.  ``idx`` is the
[T, k] top-k routing, ``w`` the [T, k] combine weights, ``x`` the [T, H]
activations as bf16 bit patterns (uint16).

Readings of points the pages leave open (each is also checked by a test):
  * routing: every slot names an expert in [0, E) and a token names each
    expert at most once; nothing is dropped and there is no capacity limit,
    so the receive buffer holds exactly T*k rows;
  * receive layout: one buffer of T*k rows, rank regions back to back in
    rank order, experts ascending inside a rank, tokens ascending inside an
    expert (a stable order by (expert, token));
  * token ownership: contiguous ceil/floor split of the tokens over ranks;
  * forwarder of (token t, node n): rank n*G + owner(t) % G, i.e. the rank
    of node n with the owner's local index; staging rows ordered by
    (forwarder, token);
  * combine: weights are applied as given (never renormalised).
"""

from __future__ import annotations

import numpy as np

from .bf16 import bf16_to_f32
from .partition import expert_partition, rank_of_expert, token_owners


class RoutingError(ValueError):
    """The top-k routing names an expert out of range or repeats one in a row."""


def validate_routing(idx: np.ndarray, num_experts: int) -> np.ndarray:
    """Check the routing reading above; return it as int64 [T, k]."""
    a = np.asarray(idx)
    if a.ndim != 2:
        raise RoutingError("topk_idx must be [T, k]")
    a = a.astype(np.int64)
    if a.size and (a.min() < 0 or a.max() >= num_experts):
        raise RoutingError("expert id outside [0, E)")
    s = np.sort(a, axis=1)
    if a.shape[1] > 1 and np.any(s[:, 1:] == s[:, :-1]):
        raise RoutingError("a token names the same expert twice")
    return a


def expert_counts(idx: np.ndarray, num_experts: int) -> np.ndarray:
    """Per-expert histogram: counts[e] = #{(t, j) : idx[t, j] == e}."""
    a = validate_routing(idx, num_experts)
    return np.bincount(a.ravel(), minlength=num_experts).astype(np.int64)


def load_aware_forwarders(node_copies: np.ndarray, G: int) -> np.ndarray:
    """fwd[s, n]: the rank of node n that forwards source s's copies for node n.

    FUSCO article, "load balancing and cross-node deduplication": forwarding
    follows the load and is spread evenly over the node's GPUs.  The pages
    give no rule; the reading taken: in each node, the sources are ranked by
    their load (copies bound for the node; more first, ties to the lower
    source) and dealt to the node's G ranks in snake order (0, 1, .., G-1,
    G-1, .., 0, 0, 1, ..).
    """
    R, N = node_copies.shape
    fwd = np.zeros((R, N), dtype=np.int64)
    for n in range(N):
        order = sorted(range(R), key=lambda s: (-int(node_copies[s, n]), s))
        for i, s in enumerate(order):
            lap, pos = divmod(i, G)
            g = pos if lap % 2 == 0 else G - 1 - pos
            fwd[s, n] = n * G + g
    return fwd


def route_plan(idx: np.ndarray, num_experts: int, num_ranks: int,
               ranks_per_node: int | None = None, forwarders: str = "static") -> dict:
    """Segment descriptors for gather-send / scatter-recv.

    FUSCO article, "core innovation": the sender reads scattered source rows
    according to segment descriptors and the receiver writes each row
    straight into its final place.  Here the descriptors are:
      counts[E], expert_offsets[E+1] (exclusive scan of counts),
      rank_offsets[R+1] = expert_offsets at each rank's first expert,
      row_src[T*k]  (receive row -> source token),
      slot_of[T, k] (token slot -> receive row; the inverse of row_src),
    plus the modelled link traffic (send_rows / send_copies [R, R],
    node_copies [R, N]) and, when there is more than one node, the
    forwarding-GPU staging descriptors of the "load balancing and cross-node
    deduplication" section (stage_src, stage_node, stage_offsets, stage_of).
    """
    a = validate_routing(idx, num_experts)
    T, k = a.shape
    E, R = num_experts, num_ranks
    G = R if ranks_per_node is None else ranks_per_node
    if G <= 0 or R % G:
        raise ValueError("ranks_per_node must divide num_ranks")
    N = R // G
    lo = expert_partition(E, R)
    rank_of = np.array([rank_of_expert(lo, e) for e in range(E)], dtype=np.int64)

    counts = np.bincount(a.ravel(), minlength=E).astype(np.int64)
    expert_offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    rank_offsets = expert_offsets[lo]

    # Stable order by expert: flat slot i = t*k + j, ties keep flat order,
    # which is token order because a token names an expert at most once.
    order = np.argsort(a.ravel(), kind="stable")
    row_src = order // max(k, 1)
    slot_flat = np.empty(T * k, dtype=np.int64)
    slot_flat[order] = np.arange(T * k, dtype=np.int64)
    slot_of = slot_flat.reshape(T, k)

    owner = token_owners(T, R)
    dest = rank_of[a]                      # [T, k] destination rank per slot
    send_rows = np.zeros((R, R), dtype=np.int64)
    np.add.at(send_rows, (np.repeat(owner, k), dest.ravel()), 1)
    present_rank = np.zeros((T, R), dtype=bool)
    present_rank[np.repeat(np.arange(T), k), dest.ravel()] = True
    send_copies = np.zeros((R, R), dtype=np.int64)
    np.add.at(send_copies, owner, present_rank.astype(np.int64))
    node = dest // G                       # [T, k] destination node per slot
    present_node = np.zeros((T, N), dtype=bool)
    present_node[np.repeat(np.arange(T), k), node.ravel()] = True
    node_copies = np.zeros((R, N), dtype=np.int64)
    np.add.at(node_copies, owner, present_node.astype(np.int64))

    plan = dict(T=T, k=k, E=E, R=R, G=G, N=N, lo=lo, rank_of=rank_of,
                counts=counts, expert_offsets=expert_offsets,
                rank_offsets=rank_offsets, row_src=row_src, slot_of=slot_of,
                owner=owner, send_rows=send_rows, send_copies=send_copies,
                node_copies=node_copies)

    # Forwarding-GPU deduplication: one staging row per distinct
    # (token, destination node); rows are ordered by (forwarder, token).  The
    # forwarder of (t, n) is rank n*G + owner(t) % G ("static"), or the
    # load-aware choice per (owner, node) above ("load_aware").
    if forwarders == "static":
        fwd_table = np.array([[n * G + s % G for n in range(N)] for s in range(R)], dtype=np.int64)
    elif forwarders == "load_aware":
        fwd_table = load_aware_forwarders(node_copies, G)
    else:
        raise ValueError(f"unknown forwarder rule {forwarders!r}")
    pt, pn = np.nonzero(present_node)      # pairs in (token, node) order
    fwd = fwd_table[owner[pt], pn] if pt.size else np.zeros(0, dtype=np.int64)
    so = np.argsort(fwd, kind="stable")    # keeps token order inside a forwarder
    stage_src = pt[so]
    stage_node = pn[so]
    D = int(stage_src.size)
    fcount = np.bincount(fwd, minlength=R).astype(np.int64)
    stage_offsets = np.concatenate([[0], np.cumsum(fcount)]).astype(np.int64)
    pos = np.full((T, N), -1, dtype=np.int64)
    pos[stage_src, stage_node] = np.arange(D, dtype=np.int64)
    stage_of = pos[np.repeat(np.arange(T), k).reshape(T, k), node]
    plan.update(num_staged=D, stage_src=stage_src, stage_node=stage_node,
                stage_offsets=stage_offsets, stage_of=stage_of, forwarders=fwd_table)
    return plan


def route_plan_banded(idx: np.ndarray, num_experts: int, num_ranks: int, band: int) -> dict:
    """Route plan of a batch cut into bands of `band` consecutive tokens.

    INC-MoE abstract: the tokens are partitioned into bands that pass through
    the dispatch, expert and combine stages one after another.  The reading
    taken: each band is routed as a batch of its own.  Band b holds tokens
    [t0, t1) = [b*band, min((b+1)*band, T)) and owns receive rows
    [t0*k, t1*k), laid out inside like a whole batch's receive buffer (ranks,
    then experts, then tokens ascending).  Returns slot_of [T, k] and
    row_src [T*k] as global rows, and per band counts [nb, E],
    expert_offsets [nb, E+1] and rank_offsets [nb, R+1] (global rows), with
    nb = max(1, ceil(T / band)).  The modelled link traffic and the token
    owners do not depend on the layout: they are the whole batch's.
    """
    if band <= 0:
        raise ValueError("band must be positive")
    a = validate_routing(idx, num_experts)
    T, k = a.shape
    nb = max(1, -(-T // band))
    plan = route_plan(a, num_experts, num_ranks)
    slot_of = np.empty((T, k), dtype=np.int64)
    row_src = np.empty(T * k, dtype=np.int64)
    counts, eoff, roff = [], [], []
    for b in range(nb):
        t0, t1 = b * band, min((b + 1) * band, T)
        p = route_plan(a[t0:t1], num_experts, num_ranks)
        base = t0 * k
        slot_of[t0:t1] = p["slot_of"] + base
        row_src[base:t1 * k] = p["row_src"] + t0
        counts.append(p["counts"])
        eoff.append(p["expert_offsets"] + base)
        roff.append(p["rank_offsets"] + base)
    plan.update(band=band, num_bands=nb, slot_of=slot_of, row_src=row_src,
                counts=np.array(counts, dtype=np.int64),
                expert_offsets=np.array(eoff, dtype=np.int64),
                rank_offsets=np.array(roff, dtype=np.int64))
    return plan


def dispatch(x: np.ndarray, plan: dict) -> np.ndarray:
    """Single-hop dispatch: recv[r] = x[row_src[r]], a bit copy of each row.

    INC-MoE abstract: dispatch moves tokens to the ranks hosting their
    experts.  FUSCO article, "core innovation": gather-send plus
    scatter-recv means each received row lands directly in its final,
    expert-contiguous position.
    """
    xa = np.asarray(x, dtype=np.uint16)
    return xa[plan["row_src"]]


def dedup_stage_a(x: np.ndarray, plan: dict) -> np.ndarray:
    """Stage A: one staging row per distinct (token, node) pair, staging[p] = x[stage_src[p]].

    FUSCO article, "load balancing and cross-node deduplication": only one
    copy of a token crosses to each destination node, through that node's
    forwarding GPU.
    """
    xa = np.asarray(x, dtype=np.uint16)
    return xa[plan["stage_src"]]


def dedup_stage_b(staging: np.ndarray, plan: dict) -> np.ndarray:
    """Stage B: intra-node fan-out, recv[slot_of[t, j]] = staging[stage_of[t, j]].

    Same section: the forwarding GPU hands the copy on over the fast
    intra-node links to every rank of its node that needs it.
    """
    s = np.asarray(staging, dtype=np.uint16)
    T, k = plan["slot_of"].shape
    recv = np.empty((T * k,) + s.shape[1:], dtype=np.uint16)
    recv[plan["slot_of"].ravel()] = s[plan["stage_of"].ravel()]
    return recv


def combine(y: np.ndarray, w: np.ndarray, plan: dict, chunk: int = 1024) -> np.ndarray:
    """out[t] = sum_j w[t, j] * y[slot_of[t, j]], summed in float64, ascending j.

    INC-MoE abstract: combine returns the expert outputs to each token's
    owner; the weighted sum over a token's k expert outputs is the MoE
    layer's output.  Returned as float64 [T, H].
    """
    ya = np.asarray(y, dtype=np.uint16)
    wa = np.asarray(w, dtype=np.float32).astype(np.float64)
    slot_of = plan["slot_of"]
    T, k = slot_of.shape
    H = ya.shape[1] if ya.ndim == 2 else 0
    out = np.zeros((T, H), dtype=np.float64)
    for s in range(0, T, chunk):
        e = min(T, s + chunk)
        acc = np.zeros((e - s, H), dtype=np.float64)
        for j in range(k):
            rows = bf16_to_f32(ya[slot_of[s:e, j]]).astype(np.float64)
            acc += wa[s:e, j:j + 1] * rows
        out[s:e] = acc
    return out


def combine_by_rank_partials(y: np.ndarray, w: np.ndarray, plan: dict) -> np.ndarray:
    """The same combine as a sum of per-rank partials (float64).

    INC-MoE abstract: combine as a ReduceScatter, i.e. every rank produces a
    partial weighted sum over the slots it hosts and the owner adds the
    partials.  partial_d[t] = sum over j with rank(idx[t, j]) == d.
    """
    ya = np.asarray(y, dtype=np.uint16)
    wa = np.asarray(w, dtype=np.float32).astype(np.float64)
    slot_of = plan["slot_of"]
    T, k = slot_of.shape
    R = plan["R"]
    H = ya.shape[1] if ya.ndim == 2 else 0
    # Rank of each receive row from the rank offsets.
    row_rank = np.searchsorted(plan["rank_offsets"], np.arange(T * k), side="right") - 1
    total = np.zeros((T, H), dtype=np.float64)
    for d in range(R):
        part = np.zeros((T, H), dtype=np.float64)
        for j in range(k):
            hit = row_rank[slot_of[:, j]] == d
            if np.any(hit):
                rows = bf16_to_f32(ya[slot_of[hit, j]]).astype(np.float64)
                part[hit] += wa[hit, j:j + 1] * rows
        total += part
    return total


def combine_hierarchical(y: np.ndarray, w: np.ndarray, plan: dict):
    """Two-hop combine over the deduplication's staging rows (float64).

    The return path of the forwarding GPU (FUSCO article, "load balancing
    and cross-node deduplication") with the ReduceScatter-style reduction of
    the INC-MoE abstract: at the forwarder, one partial per staging row
    p = (token t, node n), part[p] = sum over t's slots on n (ascending j) of
    w[t, j] * y[slot_of[t, j]]; at the owner, out[t] = sum of t's partials in
    ascending node order.  Returns (out [T, H], part [D, H]).
    """
    ya = np.asarray(y, dtype=np.uint16)
    wa = np.asarray(w, dtype=np.float32).astype(np.float64)
    slot_of, stage_of = plan["slot_of"], plan["stage_of"]
    T, k = slot_of.shape
    H = ya.shape[1] if ya.ndim == 2 else 0
    D = plan["num_staged"]
    part = np.zeros((D, H), dtype=np.float64)
    for j in range(k):
        rows = bf16_to_f32(ya[slot_of[:, j]]).astype(np.float64)
        np.add.at(part, stage_of[:, j], wa[:, j:j + 1] * rows)
    out = np.zeros((T, H), dtype=np.float64)
    node_order = np.argsort(plan["stage_node"], kind="stable")
    for p in node_order:                    # ascending node; each token has one row per node
        out[plan["stage_src"][p]] += part[p]
    return out, part


def roundtrip(x: np.ndarray, w: np.ndarray, plan: dict) -> np.ndarray:
    """Dispatch, identity expert, combine: float64 [T, H]."""
    return combine(dispatch(x, plan), w, plan)
