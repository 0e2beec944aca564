"""Pins for the oracle's ceil/floor partitions (CPU).

The oracle builds ``lo`` by prefix sums and finds a rank by linear search.
These tests check it against numbers the pages print, against the closed
form of the same split (a different formula: no prefix sums, no search), and
against the rejection rule for fewer experts than ranks.
"""

import json
import os

import numpy as np
import pytest

from oracle import expert_partition, rank_of_expert, token_owners


def closed_form_rank(e, E, R):
    # Rank of expert e when the first E % R ranks hold E // R + 1 experts.
    base, rem = E // R, E % R
    cut = rem * (base + 1)
    return np.where(e < cut, e // (base + 1), rem + (e - cut) // max(base, 1))


def test_printed_partitions(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "partition_printed.json")))
    for c in g["cases"]:
        lo = expert_partition(c["E"], c["R"])
        sizes = np.diff(lo)
        assert lo[0] == 0 and lo[-1] == c["E"], c["cite"]
        if "base" in c:
            assert sizes.min() == c["base"], c["cite"]
        if "rem" in c:
            assert int(np.sum(sizes > sizes.min())) == c["rem"] or (
                c["rem"] == 0 and sizes.min() == sizes.max()), c["cite"]
            # The larger ranges come first.
            assert np.all(np.diff(sizes) <= 0), c["cite"]
        if "sizes" in c:
            assert sizes.tolist() == c["sizes"], c["cite"]
    for c in g["errors"]:
        with pytest.raises(ValueError):
            expert_partition(c["E"], c["R"])


def test_closed_form_all_small():
    # Every 1 <= R <= E <= 256: the oracle's ranges agree with the closed form.
    for E in range(1, 257):
        e = np.arange(E)
        for R in range(1, E + 1):
            lo = expert_partition(E, R)
            d = closed_form_rank(e, E, R)
            assert np.all(lo[d] <= e) and np.all(e < lo[d + 1]), (E, R)
            sizes = np.diff(lo)
            assert sizes.max() - sizes.min() <= 1


@pytest.mark.parametrize("E,R", [(256, 7), (100, 7), (384, 5), (384, 7), (8, 2), (64, 4),
                                 (512, 509), (7, 7), (1, 1), (500, 3)])
def test_linear_search_matches_closed_form(E, R):
    lo = expert_partition(E, R)
    got = np.array([rank_of_expert(lo, e) for e in range(E)])
    assert np.array_equal(got, closed_form_rank(np.arange(E), E, R))


def test_rejects_bad_sizes():
    for E, R in [(0, 1), (1, 0), (3, 4), (2, 8)]:
        with pytest.raises(ValueError):
            expert_partition(E, R)
    with pytest.raises(ValueError):
        rank_of_expert(expert_partition(8, 2), 8)


@pytest.mark.parametrize("T,R", [(0, 3), (2, 5), (128, 2), (4096, 4), (32768, 7), (16384, 64), (10, 3)])
def test_token_owners(T, R):
    owner = token_owners(T, R)
    assert owner.shape == (T,)
    sizes = np.bincount(owner, minlength=R)
    assert sizes.sum() == T
    assert sizes.max() - sizes.min() <= 1
    assert np.all(np.diff(sizes) <= 0)          # larger shares first
    assert np.all(np.diff(owner) >= 0)          # contiguous, ascending
    np.testing.assert_array_equal(owner, closed_form_rank(np.arange(T), T, R) if T >= R
                                  else np.arange(T))
