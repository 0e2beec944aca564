"""Helpers for the GPU parity tests: run the HIP path through the C ABI and
compare with the oracle to the stated bars.

Combine tolerance.  The kernel accumulates k products with float32 fused
multiply-adds in ascending slot order starting from 0.  Each step rounds once
(relative error at most u = 2^-24 of the partial sum), so the float32 result
differs from the exact sum by at most about k*u*S, with S = sum_j |w_j*y_j|.
The bars written in the tests:
  float32 out: |gpu - ref| <= 1e-3*|ref| + k*u*S*(1 + 1e-3)
  bf16 out:    |gpu - ref| <= ulp_bf16(ref) + k*u*S*(1 + 1e-3)
i.e. 1e-3 relative, and within one bf16 unit in the last place of the exact
value once the float32 accumulation error has been allowed for (which only
matters where the k terms cancel).  ref is the oracle's float64 sum.
"""

from __future__ import annotations

import sys

import numpy as np
import torch

import combine_shuffling_amd as cs
import oracle

U32 = 2.0 ** -24


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(a: np.ndarray, dev) -> torch.Tensor:
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def bits(t: torch.Tensor) -> np.ndarray:
    return t.cpu().view(torch.int16).numpy().view(np.uint16)


def abs_scale(y: np.ndarray, w: np.ndarray, slot_of: np.ndarray) -> np.ndarray:
    ya = np.abs(oracle.bf16_to_f32(y).astype(np.float64))
    wa = np.abs(np.asarray(w, dtype=np.float64))
    return sum(wa[:, j:j + 1] * ya[slot_of[:, j]] for j in range(slot_of.shape[1]))


def ulp_bf16(ref: np.ndarray) -> np.ndarray:
    _, e = np.frexp(np.abs(ref))
    return np.ldexp(1.0, np.maximum(e - 8, -133))


def check_combine(out: np.ndarray, y: np.ndarray, w: np.ndarray, slot_of: np.ndarray,
                  out_f32: bool, what: str) -> dict:
    """out: gpu result for the tokens of slot_of (float32 or bf16 bits); y: bf16 rows."""
    k = slot_of.shape[1]
    ref = oracle.combine(y, w, {"slot_of": slot_of})
    yv = oracle.bf16_to_f32(y).astype(np.float64)
    return check_combine_values(out, ref, yv, w, slot_of, out_f32, what)


def check_combine_values(out, ref, yv, w, slot_of, out_f32, what, roundings=None) -> dict:
    """Same bars with the receive rows given as their (exact) float64 values yv.

    roundings: float32 roundings on the way to each output (default k: the
    FMA chain; the two-hop combine adds one per extra node).
    """
    k = slot_of.shape[1]
    wa = np.abs(np.asarray(w, dtype=np.float64))
    scale = sum(wa[:, j:j + 1] * np.abs(yv[slot_of[:, j]]) for j in range(k))
    acc_err = (k if roundings is None else roundings) * U32 * scale * (1 + 1e-3)
    if out_f32:
        got = out.astype(np.float64)
        bound = 1e-3 * np.abs(ref) + acc_err
    else:
        got = oracle.bf16_to_f32(out).astype(np.float64)
        bound = ulp_bf16(ref) + acc_err
    err = np.abs(got - ref)
    bad = ~(err <= bound)
    if np.any(bad):
        t, h = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: combine outside tolerance at token {t} col {h}: "
                             f"gpu={got[t, h]!r} ref={ref[t, h]!r} bound={bound[t, h]!r} "
                             f"({int(bad.sum())} elements)")
    info = {"max_abs_err": float(err.max()) if err.size else 0.0}
    if not out_f32 and err.size:
        rne = oracle.f32_to_bf16_rne(ref.astype(np.float32))
        d = oracle.bf16_ulp_distance(out, rne)
        clean = acc_err <= 0.25 * ulp_bf16(ref)
        info["max_ulp_vs_rne"] = int(d[clean].max()) if np.any(clean) else 0
        assert info["max_ulp_vs_rne"] <= 1, f"{what}: {info}"
    return info


def check_combine_chunks(out, w, slot_of, out_f32, what, ref_and_values, chunk=2048,
                         roundings=None) -> None:
    """The bars of check_combine_values on every token, chunk by chunk so that
    host memory stays bounded at full size.  ref_and_values(used, w_chunk,
    sub) returns the oracle's float64 combine of the chunk's tokens over the
    receive rows `used` (renumbered: slot_of[chunk] == used[sub]) and those
    rows' exact float64 values."""
    T = slot_of.shape[0]
    for s in range(0, T, chunk):
        e = min(T, s + chunk)
        so = slot_of[s:e]
        used = np.unique(so)
        sub = np.searchsorted(used, so)
        ref, yv = ref_and_values(used, w[s:e], sub)
        check_combine_values(out[s:e], ref, yv, w[s:e], sub, out_f32,
                             f"{what} (tokens {s}..{e - 1})", roundings)


def check_combine_all(out, y, w, slot_of, out_f32, what) -> None:
    """check_combine on every token (bf16 receive rows y), chunk by chunk."""
    check_combine_chunks(
        out, w, slot_of, out_f32, what,
        lambda used, wc, sub: (oracle.combine(y[used], wc, {"slot_of": sub}),
                               oracle.bf16_to_f32(y[used]).astype(np.float64)))


class DeviceRun:
    """One route plan + dispatch (+ combine) on the GPU through the C ABI."""

    def __init__(self, batch, dev, node_dedup=None, load_aware=False):
        wl = batch.workload
        self.wl, self.batch, self.dev = wl, batch, dev
        self.dedup = wl.node_dedup if node_dedup is None else node_dedup
        self.x = to_dev(batch.x, dev)
        self.idx = to_dev(batch.topk_idx, dev)
        self.w = to_dev(batch.topk_w, dev)
        self.plan = cs.Plan(wl.num_tokens, wl.hidden, wl.num_experts, wl.top_k, wl.num_ranks,
                            wl.ranks_per_node, self.dedup, load_aware)
        p = self.plan
        # Guard rows after every output; poisoned so unwritten rows show.
        self.recv_full = torch.full((p.recv_rows + 4, wl.hidden), -1, dtype=torch.int16, device=dev)
        self.recv = self.recv_full[: p.recv_rows]
        self.staging_full = None
        self.staging = None
        if self.dedup:
            self.staging_full = torch.full((p.staging_rows_max + 4, wl.hidden), -1,
                                           dtype=torch.int16, device=dev)
            self.staging = self.staging_full[: p.staging_rows_max]

    def route(self):
        self.plan.route(self.idx)
        return self

    def dispatch(self):
        self.plan.dispatch(self.x, self.recv, self.staging)
        return self

    def combine(self, y=None, w=None, out_dtype=torch.bfloat16):
        y = self.recv if y is None else y
        w = self.w if w is None else w
        out_full = torch.full((self.wl.num_tokens + 2, self.wl.hidden), float("nan"),
                              dtype=out_dtype, device=self.dev)
        self.plan.combine(y, w, out_full[: self.wl.num_tokens], out_dtype)
        torch.cuda.synchronize()
        assert torch.isnan(out_full[self.wl.num_tokens:].float()).all(), "combine wrote past out"
        return out_full[: self.wl.num_tokens]

    def guards_intact(self):
        torch.cuda.synchronize()
        ok = bool((self.recv_full[self.plan.recv_rows:] == -1).all())
        if self.staging_full is not None:
            ok = ok and bool((self.staging_full[self.plan.staging_rows_max:] == -1).all())
        return ok
