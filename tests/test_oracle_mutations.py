"""The oracle's pins catch plausible mistakes (CPU).

Each test plants one mistake in the oracle (a monkeypatched function: a
dropped term, a wrong index or sign, a reversed order, a rounding rule swapped
for another) and checks that the pins in tests/test_oracle_*.py fail on it.
A pin set that still passed with a planted mistake would not be pinning that
part of the oracle.  The mistakes live only inside these tests.
"""

import numpy as np
import pytest

import oracle
from oracle import bf16 as obf16, fp8 as ofp8, partition as opart, shuffle as oshuf

import test_oracle_bf16 as tb
import test_oracle_fp8 as tf
import test_oracle_partition as tp
import test_oracle_shuffle as ts


def _tiny(E, R, G, k, T, H, seed):
    """A fixed case in the format of the brute-force pins' hypothesis strategy."""
    rng = np.random.default_rng(seed)
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    x = rng.integers(0, 1 << 16, (T, H), dtype=np.uint16)
    x = np.where(np.isnan(oracle.bf16_to_f32(x)), np.uint16(0x3F80), x)
    w = rng.standard_normal((T, k)).astype(np.float32)
    return E, R, G, k, T, H, idx, x, w


CASES = [_tiny(8, 4, 2, 3, 12, 8, 1), _tiny(12, 6, 3, 5, 16, 16, 2), _tiny(5, 5, 5, 2, 9, 8, 3)]


def _brute_pins(fwd_rules=("static", "load_aware")):
    """The brute-force pins on fixed cases (their hypothesis bodies)."""
    pins = []
    for case in CASES:
        for rule in fwd_rules:
            pins.append(lambda c=case, r=rule: ts.test_plan_dispatch_combine_vs_brute.hypothesis.inner_test(c, r))
    return pins


def _hier_pins():
    return [lambda c=case: ts.test_hierarchical_combine_vs_brute.hypothesis.inner_test(c, "static")
            for case in CASES]


def _failures(pins):
    failed = 0
    for pin in pins:
        try:
            pin()
        except AssertionError:
            failed += 1
    return failed


def _patch(monkeypatch, name, fn, *modules):
    for m in modules:
        if hasattr(m, name):
            monkeypatch.setattr(m, name, fn)


def test_pins_pass_unmutated(golden_dir):
    # the same pin calls as below, on the oracle as it is
    pins = ([lambda: tb.test_golden_values(golden_dir), tb.test_matches_torch_cast,
             lambda: tp.test_printed_partitions(golden_dir), tp.test_closed_form_all_small,
             lambda: tp.test_token_owners(10, 3), lambda: ts.test_hand_example(golden_dir),
             lambda: ts.test_workload_plan_invariants("tiny"),
             ts.test_hierarchical_combine_equals_direct,
             lambda: tf.test_golden_codes(golden_dir), tf.test_block_exponent_is_smallest]
            + _brute_pins() + _hier_pins())
    assert _failures(pins) == 0


def test_bf16_truncation_instead_of_nearest_even(monkeypatch, golden_dir):
    def truncate(values):
        return (np.asarray(values, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)
    _patch(monkeypatch, "f32_to_bf16_rne", truncate, obf16, oracle, tb)
    assert _failures([lambda: tb.test_golden_values(golden_dir), tb.test_matches_torch_cast]) >= 1


def test_partition_extra_experts_on_last_ranks(monkeypatch, golden_dir):
    def last_ranks(E, R):
        if R <= 0 or E < R:
            raise ValueError("bad sizes")
        base, rem = divmod(E, R)
        sizes = [base + (1 if d >= R - rem else 0) for d in range(R)]
        return np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
    _patch(monkeypatch, "expert_partition", last_ranks, opart, oracle, oshuf, tp)
    assert _failures([lambda: tp.test_printed_partitions(golden_dir),
                      lambda: ts.test_hand_example(golden_dir)] + _brute_pins()) >= 1


def test_token_owners_extra_tokens_on_last_ranks(monkeypatch, golden_dir):
    def last_owners(T, R):
        base, rem = divmod(T, R)
        sizes = [base + (1 if d >= R - rem else 0) for d in range(R)]
        return np.repeat(np.arange(R), sizes).astype(np.int64)
    _patch(monkeypatch, "token_owners", last_owners, opart, oracle, oshuf, tp)
    assert _failures([lambda: tp.test_token_owners(10, 3), lambda: ts.test_hand_example(golden_dir)]
                     + _brute_pins()) >= 1


def test_rows_in_descending_token_order(monkeypatch, golden_dir):
    real = oshuf.route_plan

    def descending(idx, E, R, G=None, forwarders="static"):
        p = real(idx, E, R, G, forwarders=forwarders)
        a = np.asarray(idx)
        rs = p["row_src"].copy()
        off = p["expert_offsets"]
        slot = np.empty_like(p["slot_of"])
        for e in range(E):
            seg = rs[off[e]:off[e + 1]][::-1]
            rs[off[e]:off[e + 1]] = seg
            for r, t in zip(range(off[e], off[e + 1]), seg):
                slot[t, list(a[t]).index(e)] = r
        p["row_src"], p["slot_of"] = rs, slot
        return p
    _patch(monkeypatch, "route_plan", descending, oshuf, oracle)
    assert _failures([lambda: ts.test_hand_example(golden_dir),
                      lambda: ts.test_workload_plan_invariants("tiny")] + _brute_pins()) >= 1


def test_counts_drop_a_slot(monkeypatch):
    real = oshuf.route_plan

    def short_counts(idx, E, R, G=None, forwarders="static"):
        p = real(idx, E, R, G, forwarders=forwarders)
        a = np.asarray(idx)
        p["counts"] = np.bincount(a[:, :-1].ravel(), minlength=E).astype(np.int64)
        return p
    _patch(monkeypatch, "route_plan", short_counts, oshuf, oracle)
    assert _failures([lambda: ts.test_workload_plan_invariants("tiny")] + _brute_pins()) >= 1


def test_combine_weights_of_reversed_slots(monkeypatch, golden_dir):
    real = oshuf.combine
    _patch(monkeypatch, "combine", lambda y, w, p, *a: real(y, np.asarray(w)[:, ::-1], p, *a),
           oshuf, oracle)
    assert _failures([lambda: ts.test_hand_example(golden_dir)] + _brute_pins()) >= 1


def test_combine_without_weights(monkeypatch, golden_dir):
    real = oshuf.combine
    _patch(monkeypatch, "combine", lambda y, w, p, *a: real(y, np.ones_like(np.asarray(w)), p, *a),
           oshuf, oracle)
    assert _failures([lambda: ts.test_hand_example(golden_dir)] + _brute_pins()) >= 1


def test_dispatch_rows_shifted_by_one(monkeypatch):
    real = oshuf.dispatch
    _patch(monkeypatch, "dispatch", lambda x, p: np.roll(real(x, p), 1, axis=0), oshuf, oracle)
    assert _failures(_brute_pins()) >= 1


def test_staging_rows_of_the_neighbouring_token(monkeypatch):
    real = oshuf.dedup_stage_a
    _patch(monkeypatch, "dedup_stage_a", lambda x, p: np.roll(real(x, p), 1, axis=0), oshuf, oracle)
    assert _failures(_brute_pins()) >= 1


def test_hierarchical_combine_drops_a_partial(monkeypatch):
    real = oshuf.combine_hierarchical

    def drop_last(y, w, p):
        out, part = real(y, w, p)
        if part.shape[0]:
            t = p["stage_src"][-1]
            out = out.copy()
            out[t] -= part[-1]
        return out, part
    _patch(monkeypatch, "combine_hierarchical", drop_last, oshuf, oracle)
    assert _failures([ts.test_hierarchical_combine_equals_direct] + _hier_pins()) >= 1


def test_fp8_rounds_toward_zero(monkeypatch, golden_dir):
    table = ofp8.e4m3_values()
    finite = np.array([c for c in range(0x7F)], dtype=np.int64)

    def toward_zero(x):
        x = np.asarray(x, dtype=np.float64)
        mag = np.minimum(np.abs(x), 448.0)
        code = np.searchsorted(table[finite], mag, side="right") - 1
        return (code | np.where(np.signbit(x), 0x80, 0)).astype(np.uint8)
    monkeypatch.setattr(ofp8, "encode_e4m3", toward_zero)
    assert _failures([lambda: tf.test_golden_codes(golden_dir), tf.test_matches_torch_float8_cast]) >= 1


def test_fp8_block_exponent_one_too_large(monkeypatch):
    real = ofp8.block_exponent
    monkeypatch.setattr(ofp8, "block_exponent", lambda amax: real(amax) + 1)
    assert _failures([tf.test_block_exponent_is_smallest]) >= 1


@pytest.mark.parametrize("rule", ["static", "load_aware"])
def test_forwarder_rule_off_by_one(monkeypatch, rule):
    real = oshuf.route_plan

    def shifted(idx, E, R, G=None, forwarders="static"):
        p = real(idx, E, R, G, forwarders=forwarders)
        g = p["G"]
        # every forwarder moved to the next rank of its node
        p["forwarders"] = (p["forwarders"] // g) * g + (p["forwarders"] % g + 1) % g
        return p
    _patch(monkeypatch, "route_plan", shifted, oshuf, oracle)
    # cases with more than one rank per node, where the shift changes a forwarder
    pins = [lambda c=c: ts.test_plan_dispatch_combine_vs_brute.hypothesis.inner_test(c, rule)
            for c in CASES[:2]]
    assert _failures(pins) >= 1
