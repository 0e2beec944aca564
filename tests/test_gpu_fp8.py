"""GPU parity of the fp8 payload (OCP E4M3, 1x128 power-of-two block scales).

Bars: codes and block scales bit-exact against the oracle's quantization;
combine of an fp8 payload within the same tolerance as the bf16 combine,
taken against the oracle's float64 sum of the decoded values.
"""

import numpy as np
import pytest
import torch

import oracle
from oracle import fp8
from workloads import gen

from gpu_util import check_combine_chunks, check_combine_values, say, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def run_fp8(batch, dev, x_bits=None):
    import combine_shuffling_amd as cs

    wl = batch.workload
    x = batch.x if x_bits is None else x_bits
    plan = cs.Plan(wl.num_tokens, wl.hidden, wl.num_experts, wl.top_k, wl.num_ranks)
    plan.route(to_dev(batch.topk_idx, dev))
    rows = plan.recv_rows
    codes_full = torch.full((rows + 2, wl.hidden), 0x55, dtype=torch.uint8, device=dev)
    scale_full = torch.full((rows + 2, plan.scale_blocks), -1.0, dtype=torch.float32, device=dev)
    plan.dispatch_fp8(to_dev(x, dev), codes_full[:rows], scale_full[:rows])
    torch.cuda.synchronize()
    assert bool((codes_full[rows:] == 0x55).all()) and bool((scale_full[rows:] == -1.0).all())
    return plan, codes_full[:rows], scale_full[:rows]


def check_fp8(batch, dev, x_bits=None):
    wl = batch.workload
    say(f"[fp8] {wl.describe()}")
    x = batch.x if x_bits is None else x_bits
    p = oracle.route_plan(batch.topk_idx, wl.num_experts, wl.num_ranks)
    plan, codes, scales = run_fp8(batch, dev, x)
    want_c, want_e = fp8.dispatch_fp8(x, p)
    got_c = codes.cpu().numpy()
    got_s = scales.cpu().numpy().astype(np.float64)
    bad = np.argwhere(got_c != want_c)
    assert bad.size == 0, f"codes differ at {bad[:3].tolist()}: {got_c[tuple(bad[0])]:#x} vs {want_c[tuple(bad[0])]:#x}"
    assert np.array_equal(got_s, np.ldexp(1.0, want_e)), "block scales differ"
    assert np.array_equal(plan.read("slot_of").reshape(p["slot_of"].shape), p["slot_of"])
    w = to_dev(batch.topk_w, dev)
    for out_dtype in (torch.float32, torch.bfloat16):
        out = plan.combine_fp8(codes, scales, w, out_dtype=out_dtype)
        torch.cuda.synchronize()
        o = out.cpu().numpy() if out_dtype == torch.float32 else \
            out.cpu().view(torch.int16).numpy().view(np.uint16)
        check_combine_chunks(
            o, batch.topk_w, p["slot_of"], out_dtype == torch.float32, wl.name + " fp8",
            lambda used, wc, sub: (fp8.combine_fp8(want_c[used], want_e[used], wc, {"slot_of": sub}),
                                   fp8.dequantize_rows(want_c[used], want_e[used])))


@pytest.mark.parametrize("case", [
    (1, 8, 1, 1, 1), (300, 200, 8, 2, 2), (1000, 136, 24, 5, 7), (2049, 256, 64, 8, 4),
    (777, 1024, 100, 6, 7), (513, 72, 13, 13, 13),
    (900, 64, 300, 6, 10),     # 300 experts
    (700, 64, 1024, 8, 16)],   # 1024 experts
    ids=lambda c: "T{}-H{}-E{}-k{}-R{}".format(*c))
def test_fp8_small_shapes(case, dev):
    T, H, E, k, R = case
    check_fp8(gen.make_batch(gen.custom(T, H, E, k, R, seed=T + H)), dev)


@pytest.mark.parametrize("seed", range(32))
def test_fp8_random_shapes(seed, dev):
    # H a multiple of 8 up to 632: one to five scale blocks a row, rows of
    # whole and of half 16-byte code chunks; up to 1000 experts (the folded
    # scan up to 64, the separate one above)
    rng = np.random.default_rng(3000 + seed)
    E = int(rng.choice([3, 8, 17, 64, 100, 256, 1000]))
    R = int(rng.integers(1, min(E, 64) + 1))
    k = int(rng.integers(1, min(E, 16) + 1))
    T = int(rng.integers(1, 3000))
    H = int(8 * rng.integers(1, 80))
    routing = str(rng.choice(["uniform", "zipf"]))
    kw = dict(zipf_s=1.2) if routing == "zipf" else {}
    check_fp8(gen.make_batch(gen.custom(T, H, E, k, R, routing=routing, seed=seed, **kw)), dev)


@pytest.mark.parametrize("name", ["tiny", "olmoe", "qwen3", "nondiv"])
def test_fp8_workloads_full_size(name, dev):
    check_fp8(gen.make_batch(gen.get(name)), dev)


def test_fp8_zero_rows_and_tiny_values(dev):
    batch = gen.make_batch(gen.custom(400, 256, 16, 4, 4, seed=3))
    x = batch.x.copy()
    x[:50] = 0                                   # all-zero rows: scale 1, codes 0
    x[50:100] = x[50:100] & np.uint16(0x807F)    # tiny bf16 values (exponent 0): subnormal range
    x[100:150, :128] = 0                         # one zero block, one normal block
    check_fp8(batch, dev, x_bits=x)


def test_fp8_large_and_non_finite_blocks(dev):
    # Blocks whose largest magnitude is near the top of the bf16 range (e =
    # 120), and blocks holding +-inf or a NaN (e = 0, codes unspecified): the
    # scales match the oracle everywhere, the codes in every finite block.
    batch = gen.make_batch(gen.custom(300, 256, 16, 4, 4, seed=11))
    x = batch.x.copy()
    big = oracle.f32_to_bf16_rne(np.array([3.2e38, -3.2e38, 3.3895313892515355e38], np.float32))
    x[0:20, 3] = big[0]
    x[20:40, 130] = big[1]
    x[40:60, 200] = big[2]
    x[60:80, 9] = np.uint16(0x7F80)       # +inf in block 0
    x[80:100, 250] = np.uint16(0xFF80)    # -inf in block 1
    x[100:120, 64] = np.uint16(0x7FC0)    # NaN in block 0
    say("[fp8] large and non-finite blocks T300-H256-E16-k4-R4")
    p = oracle.route_plan(batch.topk_idx, 16, 4)
    plan, codes, scales = run_fp8(batch, dev, x)
    want_c, want_e = fp8.dispatch_fp8(x, p)
    got_s = scales.cpu().numpy().astype(np.float64)
    assert np.array_equal(got_s, np.ldexp(1.0, want_e)), "block scales differ"
    src = p["row_src"]
    finite = np.isfinite(oracle.bf16_to_f32(x).astype(np.float64)).reshape(300, 2, 128).all(axis=2)
    keep = np.repeat(finite[src], 128, axis=1)
    got_c = codes.cpu().numpy()
    assert np.array_equal(got_c[keep], want_c[keep]), "codes of finite blocks differ"
    assert (want_e[np.isin(src, np.arange(0, 60))] == 120).any()


def test_fp8_one_hot_combine_is_exact_decode(dev):
    batch = gen.make_batch(gen.custom(1000, 512, 32, 4, 4, seed=8))
    T, k = batch.topk_idx.shape
    p = oracle.route_plan(batch.topk_idx, 32, 4)
    plan, codes, scales = run_fp8(batch, dev)
    pick = np.random.default_rng(1).integers(0, k, T)
    w = np.zeros((T, k), dtype=np.float32)
    w[np.arange(T), pick] = 1.0
    out = plan.combine_fp8(codes, scales, to_dev(w, dev), out_dtype=torch.float32).cpu().numpy()
    c, e = fp8.dispatch_fp8(batch.x, p)
    rows = p["slot_of"][np.arange(T), pick]
    assert np.array_equal(out.astype(np.float64), fp8.dequantize_rows(c[rows], e[rows]))


def check_fp8_dedup(batch, dev, load_aware=False):
    import combine_shuffling_amd as cs

    wl = batch.workload
    T, H, k = wl.num_tokens, wl.hidden, wl.top_k
    say(f"[fp8 dedup] {wl.describe()} load_aware={load_aware}")
    p = oracle.route_plan(batch.topk_idx, wl.num_experts, wl.num_ranks, wl.ranks_per_node,
                          forwarders="load_aware" if load_aware else "static")
    sc, se, rc, re = fp8.dedup_dispatch_fp8(batch.x, p)
    plan = cs.Plan(T, H, wl.num_experts, k, wl.num_ranks, wl.ranks_per_node, True, load_aware)
    plan.route(to_dev(batch.topk_idx, dev))
    rows, smax, nb = plan.recv_rows, plan.staging_rows_max, plan.scale_blocks
    codes_full = torch.full((rows + 2, H), 0x55, dtype=torch.uint8, device=dev)
    scale_full = torch.full((rows + 2, nb), -1.0, dtype=torch.float32, device=dev)
    st8_full = torch.full((smax + 2, H), 0x55, dtype=torch.uint8, device=dev)
    sts_full = torch.full((smax + 2, nb), -1.0, dtype=torch.float32, device=dev)
    plan.dispatch_fp8(to_dev(batch.x, dev), codes_full[:rows], scale_full[:rows], st8_full[:smax],
                      sts_full[:smax])
    torch.cuda.synchronize()
    for full, n, fill in ((codes_full, rows, 0x55), (scale_full, rows, -1.0), (st8_full, smax, 0x55),
                          (sts_full, smax, -1.0)):
        assert bool((full[n:] == fill).all()), "fp8 dedup dispatch wrote past a buffer"
    D = p["num_staged"]
    assert np.array_equal(st8_full[:D].cpu().numpy(), sc), "staging codes differ"
    assert np.array_equal(sts_full[:D].cpu().numpy().astype(np.float64), np.ldexp(1.0, se))
    got_c = codes_full[:rows].cpu().numpy()
    assert np.array_equal(got_c, rc), "receive codes differ"
    assert np.array_equal(scale_full[:rows].cpu().numpy().astype(np.float64), np.ldexp(1.0, re))
    assert np.array_equal(plan.read("stage_of").reshape(T, k), p["stage_of"])
    assert np.array_equal(plan.read("stage_src")[:D], p["stage_src"])
    out = plan.combine_fp8(codes_full[:rows], scale_full[:rows], to_dev(batch.topk_w, dev),
                           out_dtype=torch.float32)
    torch.cuda.synchronize()
    check_combine_chunks(
        out.cpu().numpy(), batch.topk_w, p["slot_of"], True, wl.name + " fp8 dedup",
        lambda used, wc, sub: (fp8.combine_fp8(rc[used], re[used], wc, {"slot_of": sub}),
                               fp8.dequantize_rows(rc[used], re[used])))


@pytest.mark.parametrize("load_aware", [False, True])
@pytest.mark.parametrize("case", [
    (600, 128, 16, 4, 4, 2), (1000, 200, 64, 8, 16, 4), (777, 24, 1024, 16, 32, 8),
    (2048, 512, 256, 8, 64, 8)], ids=lambda c: "T{}-H{}-E{}-k{}-R{}-G{}".format(*c))
def test_fp8_dedup_small(case, load_aware, dev):
    T, H, E, k, R, G = case
    check_fp8_dedup(gen.make_batch(gen.custom(T, H, E, k, R, G, routing="node_limited",
                                              nodes_per_token=min(4, R // G), node_score_topn=2,
                                              seed=T + H)), dev, load_aware)


@pytest.mark.parametrize("seed", range(24))
def test_fp8_dedup_random_shapes(seed, dev):
    rng = np.random.default_rng(4000 + seed)
    E = int(rng.choice([8, 17, 64, 100, 256]))
    R = int(rng.integers(2, min(E, 64) + 1))
    G = int(rng.choice([g for g in range(1, R) if R % g == 0]))   # at least two nodes
    k = int(rng.integers(1, min(E, 16) + 1))
    T = int(rng.integers(1, 3000))
    H = int(8 * rng.integers(1, 80))
    load_aware = seed % 2 == 1 and R * (R // G) <= 1024
    check_fp8_dedup(gen.make_batch(gen.custom(T, H, E, k, R, G, seed=seed)), dev, load_aware)


def test_fp8_dedup_dsv3(dev):
    check_fp8_dedup(gen.make_batch(gen.get("dsv3")), dev)


def test_fp8_dedup_in_chunks(dev):
    # 8999 tokens of 8 staging rows of 7168 codes + 56 scales at most: the
    # fp8 dispatch runs hop 1 and hop 2 in 3 chunks, the last ragged.
    check_fp8_dedup(gen.make_batch(gen.custom(8999, 7168, 32, 8, 8, 1, seed=9)), dev)


def test_fp8_combines_without_dispatch(dev):
    import combine_shuffling_amd as cs

    batch = gen.make_batch(gen.custom(600, 128, 16, 4, 4, 2, seed=4))
    idx = to_dev(batch.topk_idx, dev)
    plan = cs.Plan(600, 128, 16, 4, 4, 2, node_dedup=True)
    plan.route(idx)
    # combine of a host-made fp8 payload straight after the route
    p = oracle.route_plan(batch.topk_idx, 16, 4, 2)
    c, e = fp8.dispatch_fp8(batch.x, p)
    out = plan.combine_fp8(to_dev(c, dev), to_dev(np.ldexp(1.0, e).astype(np.float32), dev),
                           to_dev(batch.topk_w, dev), out_dtype=torch.float32)
    ref = fp8.combine_fp8(c, e, batch.topk_w, p)
    check_combine_values(out.cpu().numpy(), ref, fp8.dequantize_rows(c, e), batch.topk_w,
                         p["slot_of"], True, "fp8 no-dispatch")
