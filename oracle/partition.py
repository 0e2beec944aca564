"""Contiguous ceil/floor partitions (oracle, test infrastructure only).

Experts to ranks -- TensorRT-LLM PR #13888 ("support non-divisible EP in MoE
alltoall"): experts are split into contiguous ranges; every rank holds
``base = E // R`` experts and the first ``E % R`` ranks hold one more (the
performance commit message prints 256 experts over 7 ranks as base 36,
remainder 4).  The host-side partition must agree with the kernel's (PR
description, "Python interface and strategy selection"), and fewer experts
than ranks is rejected with an error rather than leaving ranks empty (the
commit message on ranks with empty partitions).

Tokens to owner ranks -- the pages do not say how tokens are owned.  Reading
taken here: the same contiguous ceil/floor rule over the T tokens, which may
leave ranks without tokens when T < R (an empty batch share is legal).
"""

from __future__ import annotations

import numpy as np


def _sizes(n: int, parts: int) -> list[int]:
    base, rem = divmod(n, parts)
    return [base + (1 if d < rem else 0) for d in range(parts)]


def _prefix(sizes: list[int]) -> np.ndarray:
    lo = [0]
    for s in sizes:
        lo.append(lo[-1] + s)
    return np.asarray(lo, dtype=np.int64)


def expert_partition(num_experts: int, num_ranks: int) -> np.ndarray:
    """Range starts ``lo`` (length R+1): rank d holds experts [lo[d], lo[d+1])."""
    if num_ranks <= 0 or num_experts <= 0:
        raise ValueError("num_experts and num_ranks must be positive")
    if num_experts < num_ranks:
        raise ValueError(
            f"num_experts={num_experts} < num_ranks={num_ranks}: the split would leave "
            "ranks without experts")
    return _prefix(_sizes(num_experts, num_ranks))


def rank_of_expert(lo: np.ndarray, expert: int) -> int:
    """The rank whose range holds ``expert``, found by a linear search over ``lo``."""
    for d in range(len(lo) - 1):
        if lo[d] <= expert < lo[d + 1]:
            return d
    raise ValueError(f"expert {expert} outside [0, {lo[-1]})")


def token_owners(num_tokens: int, num_ranks: int) -> np.ndarray:
    """owner[t] for every token under the contiguous ceil/floor split of T over R."""
    if num_ranks <= 0 or num_tokens < 0:
        raise ValueError("num_ranks must be positive and num_tokens non-negative")
    lo = _prefix(_sizes(num_tokens, num_ranks))
    owner = np.empty(num_tokens, dtype=np.int64)
    for d in range(num_ranks):
        owner[lo[d]:lo[d + 1]] = d
    return owner
