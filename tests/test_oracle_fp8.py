"""Pins for the oracle's fp8 (OCP E4M3, 1x128 power-of-two block scales) payload (CPU)."""

import json
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import fp8
from workloads import gen


def test_golden_codes(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "e4m3_values.json")))
    for c in g["cases"]:
        got = int(fp8.encode_e4m3(np.array([c["value"]]))[0])
        assert got == int(c["code"], 16), c["why"]


def test_value_table_shape():
    v = fp8.e4m3_values()
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF])
    finite = v[:0x7F]
    assert np.all(np.diff(finite) > 0) and finite[-1] == 448.0
    assert np.array_equal(-v[0x80:0xFF], finite) or np.all(v[0x80:0xFF] == -finite)


def test_matches_torch_float8_cast():
    # torch's CPU cast to float8_e4m3fn rounds to nearest even inside the range.
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.uniform(-448, 448, 100000),
                        rng.standard_normal(100000) * 10.0 ** rng.integers(-4, 2, 100000)])
    x = x.astype(np.float32).astype(np.float64)
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(fp8.encode_e4m3(x), ref)


def test_decode_encode_roundtrip_all_codes():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    v = fp8.decode_e4m3(codes)
    assert np.array_equal(fp8.decode_e4m3(fp8.encode_e4m3(v)), v)


def test_block_exponent_is_smallest():
    rng = np.random.default_rng(1)
    amax = np.concatenate([np.abs(rng.standard_normal(50000)) * 10.0 ** rng.integers(-30, 30, 50000),
                           448.0 * 2.0 ** np.arange(-20, 20), [1.0, 448.0, 449.0, 224.0, 0.0]])
    amax = amax.astype(np.float32).astype(np.float64)
    e = fp8.block_exponent(amax)
    pos = amax > 0
    assert np.all(amax[pos] <= 448.0 * np.ldexp(1.0, e[pos]))
    assert np.all(amax[pos] > 448.0 * np.ldexp(1.0, e[pos] - 1))
    assert e[amax == 0].tolist() == [0]
    assert fp8.block_exponent(np.array([448.0, 449.0, 224.0, 1.0])).tolist() == [0, 1, -1, -8]


def test_block_exponent_every_bf16_magnitude():
    # Every positive finite bf16 magnitude (bit patterns 0x0001..0x7F7F), the
    # top of the range included: 2^e is the smallest power of two with
    # amax <= 448 * 2^e, unless the clamp to [-126, 127] applies (tiny blocks).
    bits = np.arange(1, 0x7F80, dtype=np.uint16)
    amax = oracle.bf16_to_f32(bits).astype(np.float64)
    e = fp8.block_exponent(amax)
    assert np.all(amax <= 448.0 * np.ldexp(1.0, e))
    small = e > -126
    assert np.all(amax[small] > 448.0 * np.ldexp(1.0, e[small] - 1))
    # 448 * 2^119 = 2.98e38 < 3.2e38 <= 448 * 2^120; 0x7F7F (3.39e38) likewise
    assert fp8.block_exponent(np.array([3.2e38, 3.3895313892515355e38])).tolist() == [120, 120]


def test_block_exponent_non_finite_blocks():
    # Reading: a block whose largest magnitude is an infinity or a NaN keeps
    # the scale 1 (e = 0); its codes are unspecified.
    assert fp8.block_exponent(np.array([np.inf, np.nan, 0.0])).tolist() == [0, 0, 0]
    row = np.zeros((3, 256), dtype=np.float32)
    row[0, :128] = 1.0
    row[0, 5] = np.inf          # block 0 of row 0: inf -> e = 0
    row[0, 128:] = 3.0
    row[1, 130] = np.nan        # block 1 of row 1: NaN -> e = 0
    row[1, :128] = -2.0
    row[2, 7] = -3.2e38         # a large finite magnitude -> e = 120
    bits = oracle.f32_to_bf16_rne(row)
    _, exps = fp8.quantize_rows(bits)
    assert exps.tolist() == [[0, -7], [-7, 0], [120, 0]]


def test_quantize_error_bound_and_block_layout():
    wl = gen.custom(300, 200, 8, 2, 2)        # H=200: blocks of 128 and 72
    b = gen.make_batch(wl)
    codes, exps = fp8.quantize_rows(b.x)
    assert codes.shape == (300, 200) and exps.shape == (300, 2)
    x = oracle.bf16_to_f32(b.x).astype(np.float64)
    deq = fp8.dequantize_rows(codes, exps)
    scale = np.repeat(np.ldexp(1.0, exps), 128, axis=1)[:, :200]
    # half a unit in the last place: 2^-4 relative for normals, 2^-10 * scale below
    assert np.all(np.abs(deq - x) <= 2.0 ** -4 * np.abs(x) + 2.0 ** -10 * scale)
    # every block's largest element lands in (224, 448] after scaling
    for blk in range(2):
        m = np.max(np.abs(x[:, blk * 128:(blk + 1) * 128]), axis=1) * np.ldexp(1.0, -exps[:, blk])
        assert np.all((m > 224) & (m <= 448))


def test_dispatch_fp8_is_row_gather_of_quantized_rows():
    wl = gen.custom(500, 256, 16, 4, 4, seed=2)
    b = gen.make_batch(wl)
    p = oracle.route_plan(b.topk_idx, 16, 4)
    codes, exps = fp8.dispatch_fp8(b.x, p)
    qc, qe = fp8.quantize_rows(oracle.dispatch(b.x, p))   # quantizing received rows gives the same
    assert np.array_equal(codes, qc) and np.array_equal(exps, qe)


def test_combine_fp8_one_hot_and_brute():
    wl = gen.custom(64, 256, 8, 3, 2, seed=5)
    b = gen.make_batch(wl)
    p = oracle.route_plan(b.topk_idx, 8, 2)
    codes, exps = fp8.dispatch_fp8(b.x, p)
    T, k = b.topk_idx.shape
    w = np.zeros((T, k), dtype=np.float32)
    w[:, 1] = 1.0
    out = fp8.combine_fp8(codes, exps, w, p)
    assert np.array_equal(out, fp8.dequantize_rows(codes[p["slot_of"][:, 1]], exps[p["slot_of"][:, 1]]))
    out = fp8.combine_fp8(codes, exps, b.topk_w, p)
    deq = fp8.dequantize_rows(codes, exps)
    for t in range(0, T, 7):
        for h in range(0, 256, 31):
            acc = 0.0
            for j in range(k):
                acc += float(b.topk_w[t, j]) * float(deq[p["slot_of"][t, j], h])
            assert out[t, h] == acc


def test_fp8_combine_within_quantization_bound():
    # Against the full-precision path the fp8 path may differ by at most the
    # half-ulp quantization error of each term: sum_j |w_j| (2^-4 |y_j| + 2^-10 * 2^e_j).
    # (The pages check their fp8 case at rtol 0.02, atol 0.15; E4M3's own
    # half-ulp is 2^-4 relative, so that check cannot hold for every element of
    # an N(0,1) payload -- 4.25 rounds to 4.0 -- and is context only.)
    b = gen.make_batch(gen.get("olmoe"))
    p = oracle.route_plan(b.topk_idx, 64, 4)
    codes, exps = fp8.dispatch_fp8(b.x, p)
    sl = slice(0, 512)
    so = p["slot_of"][sl]
    q = fp8.combine_fp8(codes, exps, b.topk_w[sl], {"slot_of": so})
    y = oracle.bf16_to_f32(oracle.dispatch(b.x, p)).astype(np.float64)
    ref = oracle.combine(oracle.dispatch(b.x, p), b.topk_w[sl], {"slot_of": so})
    w = np.abs(b.topk_w[sl].astype(np.float64))
    scale = np.repeat(np.ldexp(1.0, exps), 128, axis=1)
    bound = sum(w[:, j:j + 1] * (2.0 ** -4 * np.abs(y[so[:, j]]) + 2.0 ** -10 * scale[so[:, j]])
                for j in range(so.shape[1]))
    assert np.all(np.abs(q - ref) <= bound * (1 + 1e-9))


@pytest.mark.parametrize("fwd", ["static", "load_aware"])
def test_dedup_fp8_fan_out_equals_single_hop(fwd):
    # The staging hop carries each (token, node) once; after the fan-out every
    # receive row holds exactly the single-hop payload.
    b = gen.make_batch(gen.custom(900, 200, 64, 8, 16, 4, routing="node_limited",
                                  nodes_per_token=2, node_score_topn=2, seed=6))
    p = oracle.route_plan(b.topk_idx, 64, 16, 4, forwarders=fwd)
    sc, se, rc, re = fp8.dedup_dispatch_fp8(b.x, p)
    c1, e1 = fp8.dispatch_fp8(b.x, p)
    assert np.array_equal(rc, c1) and np.array_equal(re, e1)
    assert sc.shape == (p["num_staged"], 200) and se.shape == (p["num_staged"], 2)
    # each staging row decodes to its token within half an E4M3 step
    x = oracle.bf16_to_f32(b.x).astype(np.float64)[p["stage_src"]]
    scale = np.repeat(np.ldexp(1.0, se), 128, axis=1)[:, :200]
    assert np.all(np.abs(fp8.dequantize_rows(sc, se) - x) <= 2.0 ** -4 * np.abs(x) + 2.0 ** -10 * scale)
    # fewer staged rows than receive rows: the hop saves payload
    assert p["num_staged"] < rc.shape[0]
