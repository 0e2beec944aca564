"""The largest batch the 32-bit row indices allow (GPU, 90 to 130 GB of HBM).

T*k = 2,147,479,536 receive rows, just under the library's limit of
2**31 - 4097 (32-bit row indices, with a margin for the last block of a
launch): every row index, every slot and every 64-bit byte offset of the
single-hop path is exercised at the top of its range, and the batch takes
several launches of at most 2**24 wave-items each.  The oracle cannot run at this size, so the expected
results come from closed forms of a round-robin routing (the oracle's own
round-robin pin, tests/test_oracle_shuffle.py, checks the same closed form):
idx[t, j] = (t*k + j) mod E with E dividing T*k gives every expert T*k/E rows,
and the flat slot f = t*k + j lands on row (f mod E) * T*k/E + f div E.
Each 16-byte token row carries its token id in four bf16 integers (7 bits
each, exact), so every receive row names the token it came from; weights
1/k (k a power of two) make the combine return x bit for bit.
"""

import pytest
import torch

import combine_shuffling_amd as cs

from gpu_util import say

pytestmark = pytest.mark.gpu

E, K, R, H = 16, 8, 2, 8
LIMIT = 2 ** 31 - 1 - 4096                 # the library's bound on T*k
T = ((LIMIT - 1) // K) // 2 * 2            # even, so E divides T*K
ROWS = T * K
PER_EXPERT = ROWS // E
STEP = 1 << 26                              # rows checked per pass


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    free, _ = torch.cuda.mem_get_info()
    if free < 120 * (1 << 30):
        pytest.skip("needs about 100 GiB of free device memory")
    return torch.device("cuda:0")


def token_rows(t: torch.Tensor) -> torch.Tensor:
    """[n, 8] bf16 rows: t in four 7-bit pieces, then 1.0 four times."""
    pieces = torch.stack([(t >> (7 * i)) & 127 for i in range(4)], dim=1).to(torch.float32)
    ones = torch.ones((t.numel(), 4), dtype=torch.float32, device=t.device)
    return torch.cat([pieces, ones], dim=1).to(torch.bfloat16)


def row_token(rows: torch.Tensor) -> torch.Tensor:
    """Inverse of token_rows (int64 token ids)."""
    p = rows[:, :4].to(torch.float32).to(torch.int64)
    return p[:, 0] | (p[:, 1] << 7) | (p[:, 2] << 14) | (p[:, 3] << 21)


def test_maximum_size_round_robin(dev):
    assert ROWS < LIMIT and ROWS % E == 0
    say(f"[max size] T={T} k={K} E={E} R={R} H={H}: {ROWS} receive rows")
    x = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    for a in range(0, T, STEP):
        b = min(T, a + STEP)
        x[a:b] = token_rows(torch.arange(a, b, device=dev))
    idx = ((torch.arange(T, device=dev, dtype=torch.int64)[:, None] * K
            + torch.arange(K, device=dev)[None, :]) % E).to(torch.int32)
    w = torch.full((T, K), 1.0 / K, dtype=torch.float32, device=dev)

    plan = cs.route_plan(idx, E, R, H)
    recv, _ = cs.dispatch(plan, x)
    out = cs.combine(plan, recv, w)
    torch.cuda.synchronize()
    assert plan.status() == 0
    counts = plan.read("counts")
    assert counts.tolist() == [PER_EXPERT] * E

    # receive row r holds the token whose flat slot lands there
    for a in range(0, ROWS, STEP):
        b = min(ROWS, a + STEP)
        r = torch.arange(a, b, device=dev, dtype=torch.int64)
        e = r // PER_EXPERT
        f = (r - e * PER_EXPERT) * E + e
        assert torch.equal(row_token(recv[a:b]), f // K), f"receive rows [{a}, {b})"
    # identity expert and weights 1/k: the combine returns x exactly
    for a in range(0, T, STEP):
        b = min(T, a + STEP)
        assert torch.equal(out[a:b].view(torch.int16), x[a:b].view(torch.int16)), f"out [{a}, {b})"


def test_maximum_size_node_dedup(dev):
    """The same batch over two one-rank nodes with node deduplication.

    Experts 0-7 sit on node 0 and 8-15 on node 1, so the round-robin routing
    sends even tokens to node 0 only and odd tokens to node 1 only: one
    staging row per token (D = T), forwarder 0 holding the even tokens in
    order and forwarder 1 the odd ones, and the same receive rows as the
    single hop.  The hierarchical combine (one fp32 partial per staging row,
    then the sum over nodes) returns x bit for bit too."""
    free, _ = torch.cuda.mem_get_info()
    if free < 160 * (1 << 30):
        pytest.skip("needs about 150 GiB of free device memory")
    say(f"[max size, dedup] T={T} k={K} E={E} R={R} G=1: {ROWS} receive rows, {T} staging rows")
    x = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    for a in range(0, T, STEP):
        b = min(T, a + STEP)
        x[a:b] = token_rows(torch.arange(a, b, device=dev))
    idx = ((torch.arange(T, device=dev, dtype=torch.int64)[:, None] * K
            + torch.arange(K, device=dev)[None, :]) % E).to(torch.int32)
    w = torch.full((T, K), 1.0 / K, dtype=torch.float32, device=dev)

    plan = cs.route_plan(idx, E, R, H, ranks_per_node=1, node_dedup=True)
    recv, staging = cs.dispatch(plan, x)
    out = cs.combine(plan, recv, w)
    torch.cuda.synchronize()
    assert plan.status() == 0
    assert int(plan.read("num_staged")[0]) == T
    assert plan.read("stage_offsets").tolist() == [0, T // 2, T]

    half = T // 2
    for a in range(0, T, STEP):
        b = min(T, a + STEP)
        q = torch.arange(a, b, device=dev, dtype=torch.int64)
        want = torch.where(q < half, 2 * q, 2 * (q - half) + 1)
        assert torch.equal(row_token(staging[a:b]), want), f"staging rows [{a}, {b})"
    for a in range(0, ROWS, STEP):
        b = min(ROWS, a + STEP)
        r = torch.arange(a, b, device=dev, dtype=torch.int64)
        e = r // PER_EXPERT
        f = (r - e * PER_EXPERT) * E + e
        assert torch.equal(row_token(recv[a:b]), f // K), f"receive rows [{a}, {b})"
    for a in range(0, T, STEP):
        b = min(T, a + STEP)
        assert torch.equal(out[a:b].view(torch.int16), x[a:b].view(torch.int16)), f"out [{a}, {b})"
    del out
    out_h = cs.combine_hier(plan, recv, w)
    torch.cuda.synchronize()
    for a in range(0, T, STEP):
        b = min(T, a + STEP)
        assert torch.equal(out_h[a:b].view(torch.int16), x[a:b].view(torch.int16)), \
            f"hierarchical out [{a}, {b})"


def test_maximum_size_fp8(dev):
    """The same batch with the fp8 payload.  A row now holds its token id in
    seven base-16 digits plus a 15, so every 8-element block has amax 15,
    scale 2^-4 and exact E4M3 codes (a digit times 16 needs at most four
    significant bits): the codes name each row's token, and the combine
    still returns x bit for bit."""
    free, _ = torch.cuda.mem_get_info()
    if free < 110 * (1 << 30):
        pytest.skip("needs about 100 GiB of free device memory")
    say(f"[max size, fp8] T={T} k={K} E={E} R={R}: {ROWS} receive rows")

    def rows16(t):
        d = torch.stack([(t >> (4 * i)) & 15 for i in range(7)] + [torch.full_like(t, 15)], dim=1)
        return d.to(torch.float32).to(torch.bfloat16)

    table = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn) \
        .to(torch.float32).to(dev)
    x = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    for a in range(0, T, STEP):
        b = min(T, a + STEP)
        x[a:b] = rows16(torch.arange(a, b, device=dev))
    idx = ((torch.arange(T, device=dev, dtype=torch.int64)[:, None] * K
            + torch.arange(K, device=dev)[None, :]) % E).to(torch.int32)
    w = torch.full((T, K), 1.0 / K, dtype=torch.float32, device=dev)

    plan = cs.route_plan(idx, E, R, H)
    codes, scales = cs.dispatch_fp8(plan, x)
    out = cs.combine_fp8(plan, codes, scales, w)
    torch.cuda.synchronize()
    assert plan.status() == 0
    assert scales.shape == (ROWS, 1)

    for a in range(0, ROWS, STEP):
        b = min(ROWS, a + STEP)
        assert torch.all(scales[a:b] == 1.0 / 16), f"scales [{a}, {b})"
        digits = (table[codes[a:b].long()] * (1.0 / 16)).to(torch.int64)
        got = sum(digits[:, i] << (4 * i) for i in range(7))
        r = torch.arange(a, b, device=dev, dtype=torch.int64)
        e = r // PER_EXPERT
        f = (r - e * PER_EXPERT) * E + e
        assert torch.equal(got, f // K), f"receive rows [{a}, {b})"
        assert torch.all(digits[:, 7] == 15)
    for a in range(0, T, STEP):
        b = min(T, a + STEP)
        assert torch.equal(out[a:b].view(torch.int16), x[a:b].view(torch.int16)), f"out [{a}, {b})"
