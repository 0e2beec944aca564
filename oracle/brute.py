"""Pure-Python re-derivation of the shuffle for tiny inputs (test infrastructure only).

Nested loops over lists, no numpy in the arithmetic, so that a slip in the
vectorised oracle (a transposed index, a wrong scan, an unstable sort) shows
up as a disagreement.  Same definitions and readings as ``oracle.shuffle``.
"""

from __future__ import annotations

import struct


def _part_starts(n: int, parts: int) -> list[int]:
    # Walk the ranks, handing out one extra element while the remainder lasts.
    starts, pos, extra = [0], 0, n - (n // parts) * parts
    for _ in range(parts):
        take = n // parts
        if extra > 0:
            take += 1
            extra -= 1
        pos += take
        starts.append(pos)
    return starts


def plan(idx: list[list[int]], E: int, R: int, G: int, forwarders: str = "static") -> dict:
    T = len(idx)
    k = len(idx[0]) if T else 0
    estarts = _part_starts(E, R)
    tstarts = _part_starts(T, R)

    def rank_of(e):
        d = 0
        while not (estarts[d] <= e < estarts[d + 1]):
            d += 1
        return d

    def owner(t):
        d = 0
        while not (tstarts[d] <= t < tstarts[d + 1]):
            d += 1
        return d

    counts = [0] * E
    for t in range(T):
        for j in range(k):
            counts[idx[t][j]] += 1
    offsets = [0]
    for e in range(E):
        offsets.append(offsets[-1] + counts[e])
    rank_offsets = [offsets[estarts[d]] for d in range(R + 1)]

    # Rows in (expert, token) order.
    row_src, slot_of = [], [[None] * k for _ in range(T)]
    for e in range(E):
        for t in range(T):
            for j in range(k):
                if idx[t][j] == e:
                    slot_of[t][j] = len(row_src)
                    row_src.append(t)

    send_rows = [[0] * R for _ in range(R)]
    send_copies = [[0] * R for _ in range(R)]
    N = R // G
    node_copies = [[0] * N for _ in range(R)]
    for t in range(T):
        s = owner(t)
        ranks = set()
        nodes = set()
        for j in range(k):
            d = rank_of(idx[t][j])
            send_rows[s][d] += 1
            ranks.add(d)
            nodes.add(d // G)
        for d in ranks:
            send_copies[s][d] += 1
        for n in nodes:
            node_copies[s][n] += 1

    # Forwarder of each (source, node): static same-local-index, or the
    # load-aware snake deal of sources ranked by load.
    fwd = [[n * G + s % G for n in range(N)] for s in range(R)]
    if forwarders == "load_aware":
        for n in range(N):
            ranked = []
            for s in range(R):
                # insert s after every source with more load, or equal load and lower id
                at = 0
                while at < len(ranked) and (node_copies[ranked[at]][n] > node_copies[s][n] or
                                            (node_copies[ranked[at]][n] == node_copies[s][n]
                                             and ranked[at] < s)):
                    at += 1
                ranked.insert(at, s)
            for i, s in enumerate(ranked):
                lap, posn = i // G, i % G
                fwd[s][n] = n * G + (posn if lap % 2 == 0 else G - 1 - posn)

    # Forwarder staging: walk forwarders in order, then tokens.
    stage_src, stage_node, stage_offsets = [], [], [0]
    pos = {}
    for f in range(R):
        n = f // G
        for t in range(T):
            if fwd[owner(t)][n] != f:
                continue
            if any(rank_of(idx[t][j]) // G == n for j in range(k)):
                pos[(t, n)] = len(stage_src)
                stage_src.append(t)
                stage_node.append(n)
        stage_offsets.append(len(stage_src))
    stage_of = [[pos[(t, rank_of(idx[t][j]) // G)] for j in range(k)] for t in range(T)]

    return dict(counts=counts, expert_offsets=offsets, rank_offsets=rank_offsets,
                row_src=row_src, slot_of=slot_of, send_rows=send_rows,
                send_copies=send_copies, node_copies=node_copies,
                stage_src=stage_src, stage_node=stage_node,
                stage_offsets=stage_offsets, stage_of=stage_of,
                num_staged=len(stage_src), forwarders=fwd)


def dispatch(x: list[list[int]], p: dict) -> list[list[int]]:
    T = len(p["slot_of"])
    k = len(p["slot_of"][0]) if T else 0
    recv = [None] * (T * k)
    for t in range(T):
        for j in range(k):
            recv[p["slot_of"][t][j]] = list(x[t])
    return recv


def bf16_value(bits: int) -> float:
    return struct.unpack("<f", struct.pack("<I", (bits & 0xFFFF) << 16))[0]


def combine(y: list[list[int]], w: list[list[float]], p: dict) -> list[list[float]]:
    T = len(p["slot_of"])
    k = len(p["slot_of"][0]) if T else 0
    H = len(y[0]) if y else 0
    out = []
    for t in range(T):
        row = []
        for h in range(H):
            acc = 0.0
            for j in range(k):
                acc += float(w[t][j]) * bf16_value(y[p["slot_of"][t][j]][h])
            row.append(acc)
        out.append(row)
    return out


def combine_hierarchical(y: list[list[int]], w: list[list[float]], p: dict) -> list[list[float]]:
    """Partials per (token, node), then the sum over the token's nodes in node order."""
    T = len(p["slot_of"])
    k = len(p["slot_of"][0]) if T else 0
    H = len(y[0]) if y else 0
    out = []
    for t in range(T):
        nodes = sorted(set(p["stage_node"][p["stage_of"][t][j]] for j in range(k)))
        row = []
        for h in range(H):
            acc = 0.0
            for n in nodes:
                part = 0.0
                for j in range(k):
                    if p["stage_node"][p["stage_of"][t][j]] == n:
                        part += float(w[t][j]) * bf16_value(y[p["slot_of"][t][j]][h])
                acc += part
            row.append(acc)
        out.append(row)
    return out


def plan_banded(idx: list[list[int]], E: int, R: int, band: int) -> dict:
    """Each band of `band` consecutive tokens routed on its own, rows numbered on from t0*k."""
    T = len(idx)
    k = len(idx[0]) if T else 0
    estarts = _part_starts(E, R)
    nb = max(1, (T + band - 1) // band)
    slot_of = [[None] * k for _ in range(T)]
    row_src = [None] * (T * k)
    counts, eoff, roff = [], [], []
    for b in range(nb):
        t0, t1 = b * band, min((b + 1) * band, T)
        nxt = t0 * k
        c = [0] * E
        offs = []
        for e in range(E):
            offs.append(nxt)
            for t in range(t0, t1):
                for j in range(k):
                    if idx[t][j] == e:
                        slot_of[t][j] = nxt
                        row_src[nxt] = t
                        nxt += 1
                        c[e] += 1
        offs.append(nxt)
        counts.append(c)
        eoff.append(offs)
        roff.append([offs[estarts[d]] for d in range(R + 1)])
    return dict(slot_of=slot_of, row_src=row_src, counts=counts, expert_offsets=eoff,
                rank_offsets=roff, num_bands=nb)
