"""MI355X (gfx950) MoE expert-parallel shuffle.

A thin binding over the C ABI of ``libmoeshuffle.so`` (include/moe_shuffle.h):
the same calls, with torch tensors for device memory and torch's current
stream.  Every step of the shuffle runs in the library's HIP kernels; this
module only checks shapes and passes pointers.

    plan = route_plan(topk_idx, num_experts=E, num_ranks=R, hidden=H,
                      ranks_per_node=G, node_dedup=False)
    recv, staging = dispatch(plan, x)           # x: [T, H] bf16 on the GPU
    out = combine(plan, y, topk_w)              # y: [T*k, H] bf16, receive layout

Banded plans (band_tokens > 0) route each band of consecutive tokens as its
own batch; ``Plan.pipeline`` runs route, dispatch and combine of every band
in one persistent launch.
"""

from __future__ import annotations

import ctypes

import numpy as np
import torch

from . import _abi
from ._abi import MoeError, ITEM  # noqa: F401

__all__ = ["Plan", "MoeError", "expert_partition", "route_plan", "dispatch", "combine",
           "dispatch_fp8", "combine_fp8", "combine_hier", "pipeline"]


def expert_partition(num_experts: int, num_ranks: int) -> list[int]:
    """moe_expert_partition: rank d holds experts [lo[d], lo[d+1])."""
    lo = (ctypes.c_int32 * (num_ranks + 1))() if num_ranks > 0 else (ctypes.c_int32 * 1)()
    _abi.check(_abi.lib().moe_expert_partition(num_experts, num_ranks, lo), "moe_expert_partition")
    return list(lo)


def _stream_handle(device: torch.device, stream) -> ctypes.c_void_p:
    s = torch.cuda.current_stream(device) if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t: torch.Tensor | None) -> ctypes.c_void_p:
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


def _need(t: torch.Tensor, shape, dtypes, name: str, device) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype not in dtypes:
        raise ValueError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


_BF16_LIKE = (torch.bfloat16, torch.int16, torch.uint16)


class Plan:
    """Owns one moe_plan (host) and, once routed, its device workspace tensor."""

    def __init__(self, num_tokens: int, hidden: int, num_experts: int, top_k: int,
                 num_ranks: int, ranks_per_node: int | None = None, node_dedup: bool = False,
                 load_aware_forwarders: bool = False, band_tokens: int = 0):
        G = num_ranks if ranks_per_node is None else ranks_per_node
        flags = (_abi.FLAG_NODE_DEDUP if node_dedup else 0) | \
            (_abi.FLAG_LOAD_AWARE_FORWARDERS if load_aware_forwarders else 0)
        self.cfg = _abi.MoeConfig(num_tokens, hidden, num_experts, top_k, num_ranks, G, flags,
                                  band_tokens)
        self._lib = _abi.lib()
        h = ctypes.c_void_p()
        _abi.check(self._lib.moe_plan_create(ctypes.byref(self.cfg), ctypes.byref(h)),
                   "moe_plan_create")
        self._h = h
        self.T, self.H, self.E, self.k = num_tokens, hidden, num_experts, top_k
        self.R, self.G, self.N = num_ranks, G, num_ranks // G
        self.node_dedup = node_dedup
        self.workspace_bytes = int(self._lib.moe_plan_workspace_bytes(h))
        self.recv_rows = int(self._lib.moe_plan_recv_rows(h))
        self.staging_rows_max = int(self._lib.moe_plan_staging_rows_max(h))
        self.scale_blocks = int(self._lib.moe_plan_scale_blocks(h))
        self.bands = int(self._lib.moe_plan_bands(h))
        # tokens per chunk of the chunked calls of a node-deduplicated plan
        self.chunk_tokens = {call: int(self._lib.moe_plan_chunk_tokens(h, i))
                             for i, call in enumerate(("dispatch", "dispatch_fp8", "combine_hier"))}
        self.workspace = None
        self.topk_idx = None
        self.device = None

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value:
            self._lib.moe_plan_destroy(h)
            self._h = None

    # -- moe_route_plan
    def route(self, topk_idx: torch.Tensor, workspace: torch.Tensor | None = None, stream=None):
        dev = topk_idx.device
        _need(topk_idx, (self.T, self.k), (torch.int32,), "topk_idx", dev)
        if workspace is None:
            if self.workspace is None or self.workspace.device != dev:
                self.workspace = torch.empty(self.workspace_bytes, dtype=torch.uint8, device=dev)
            workspace = self.workspace
        elif workspace.numel() * workspace.element_size() < self.workspace_bytes:
            raise ValueError("workspace too small")
        self.workspace, self.topk_idx, self.device = workspace, topk_idx, dev
        _abi.check(self._lib.moe_route_plan(self._h, _ptr(topk_idx), _ptr(workspace),
                                            _stream_handle(dev, stream)), "moe_route_plan")
        return self

    # -- moe_route_plan_static
    def route_static(self, topk_idx: torch.Tensor, stream=None):
        """moe_route_plan_static: the route plan on the library's per-device
        static workspace; allocates nothing.  Plans routed this way on one GPU
        share that workspace: the last one routed is the one that holds it."""
        dev = topk_idx.device
        _need(topk_idx, (self.T, self.k), (torch.int32,), "topk_idx", dev)
        self.workspace, self.topk_idx, self.device = None, topk_idx, dev
        _abi.check(self._lib.moe_route_plan_static(self._h, _ptr(topk_idx),
                                                   _stream_handle(dev, stream)),
                   "moe_route_plan_static")
        return self

    # -- moe_pipeline
    def pipeline(self, topk_idx: torch.Tensor, x: torch.Tensor, topk_w: torch.Tensor,
                 recv: torch.Tensor | None = None, out: torch.Tensor | None = None,
                 out_dtype: torch.dtype = torch.bfloat16, workspace: torch.Tensor | None = None,
                 stream=None):
        """Route, dispatch and combine (identity expert) of every band in one launch.

        Returns (recv [T*k, H], out [T, H]); the plan is routed afterwards."""
        dev = topk_idx.device
        _need(topk_idx, (self.T, self.k), (torch.int32,), "topk_idx", dev)
        _need(x, (self.T, self.H), _BF16_LIKE, "x", dev)
        _need(topk_w, (self.T, self.k), (torch.float32,), "topk_w", dev)
        if out_dtype not in (torch.bfloat16, torch.float32):
            raise ValueError("out_dtype must be torch.bfloat16 or torch.float32")
        if recv is None:
            recv = torch.empty((self.recv_rows, self.H), dtype=x.dtype, device=dev)
        _need(recv, (self.recv_rows, self.H), _BF16_LIKE, "recv", dev)
        if out is None:
            out = torch.empty((self.T, self.H), dtype=out_dtype, device=dev)
        _need(out, (self.T, self.H), (out_dtype,), "out", dev)
        if workspace is None:
            if self.workspace is None or self.workspace.device != dev:
                self.workspace = torch.empty(self.workspace_bytes, dtype=torch.uint8, device=dev)
            workspace = self.workspace
        elif workspace.numel() * workspace.element_size() < self.workspace_bytes:
            raise ValueError("workspace too small")
        self.workspace, self.topk_idx, self.device = workspace, topk_idx, dev
        code = _abi.OUT_F32 if out_dtype == torch.float32 else _abi.OUT_BF16
        _abi.check(self._lib.moe_pipeline(self._h, _ptr(topk_idx), _ptr(workspace), _ptr(x),
                                          _ptr(recv), _ptr(topk_w), _ptr(out), code,
                                          _stream_handle(dev, stream)), "moe_pipeline")
        return recv, out

    # -- moe_dispatch
    def dispatch(self, x: torch.Tensor, recv: torch.Tensor | None = None,
                 staging: torch.Tensor | None = None, stream=None):
        dev = self.device
        if dev is None:
            raise MoeError(_abi.ERR_PLAN_NOT_ROUTED, "dispatch")
        _need(x, (self.T, self.H), _BF16_LIKE, "x", dev)
        if recv is None:
            recv = torch.empty((self.recv_rows, self.H), dtype=x.dtype, device=dev)
        _need(recv, (self.recv_rows, self.H), _BF16_LIKE, "recv", dev)
        if self.node_dedup:
            if staging is None:
                staging = torch.empty((self.staging_rows_max, self.H), dtype=x.dtype, device=dev)
            _need(staging, (self.staging_rows_max, self.H), _BF16_LIKE, "staging", dev)
        _abi.check(self._lib.moe_dispatch(self._h, _ptr(x), _ptr(recv), _ptr(staging),
                                          _stream_handle(dev, stream)), "moe_dispatch")
        return recv, staging

    # -- moe_combine
    def combine(self, y: torch.Tensor, topk_w: torch.Tensor, out: torch.Tensor | None = None,
                out_dtype: torch.dtype = torch.bfloat16, stream=None) -> torch.Tensor:
        dev = self.device
        if dev is None:
            raise MoeError(_abi.ERR_PLAN_NOT_ROUTED, "combine")
        _need(y, (self.recv_rows, self.H), _BF16_LIKE, "y", dev)
        _need(topk_w, (self.T, self.k), (torch.float32,), "topk_w", dev)
        if out_dtype not in (torch.bfloat16, torch.float32):
            raise ValueError("out_dtype must be torch.bfloat16 or torch.float32")
        if out is None:
            out = torch.empty((self.T, self.H), dtype=out_dtype, device=dev)
        _need(out, (self.T, self.H), (out_dtype,), "out", dev)
        code = _abi.OUT_F32 if out_dtype == torch.float32 else _abi.OUT_BF16
        _abi.check(self._lib.moe_combine(self._h, _ptr(y), _ptr(topk_w), _ptr(out), code,
                                         _stream_handle(dev, stream)), "moe_combine")
        return out

    # -- moe_combine_hier
    def combine_hier(self, y: torch.Tensor, topk_w: torch.Tensor,
                     partials: torch.Tensor | None = None, out: torch.Tensor | None = None,
                     out_dtype: torch.dtype = torch.bfloat16, stream=None) -> torch.Tensor:
        """Two-hop combine of a node-deduplicated plan (fp32 partial per staging row)."""
        dev = self.device
        if dev is None:
            raise MoeError(_abi.ERR_PLAN_NOT_ROUTED, "combine_hier")
        _need(y, (self.recv_rows, self.H), _BF16_LIKE, "y", dev)
        _need(topk_w, (self.T, self.k), (torch.float32,), "topk_w", dev)
        if out_dtype not in (torch.bfloat16, torch.float32):
            raise ValueError("out_dtype must be torch.bfloat16 or torch.float32")
        if partials is None:
            partials = torch.empty((self.staging_rows_max, self.H), dtype=torch.float32, device=dev)
        _need(partials, (self.staging_rows_max, self.H), (torch.float32,), "partials", dev)
        if out is None:
            out = torch.empty((self.T, self.H), dtype=out_dtype, device=dev)
        _need(out, (self.T, self.H), (out_dtype,), "out", dev)
        code = _abi.OUT_F32 if out_dtype == torch.float32 else _abi.OUT_BF16
        _abi.check(self._lib.moe_combine_hier(self._h, _ptr(y), _ptr(topk_w), _ptr(partials),
                                              _ptr(out), code, _stream_handle(dev, stream)),
                   "moe_combine_hier")
        return out

    # -- moe_dispatch_fp8
    def dispatch_fp8(self, x: torch.Tensor, recv8: torch.Tensor | None = None,
                     recv_scale: torch.Tensor | None = None, staging8: torch.Tensor | None = None,
                     staging_scale: torch.Tensor | None = None, stream=None):
        """fp8 payload: returns (codes uint8 [T*k, H], block scales float32 [T*k, nb]).

        With node deduplication the codes and scales pass through staging rows
        (staging8 [staging_rows_max, H] uint8, staging_scale [.., nb] float32)."""
        dev = self.device
        if dev is None:
            raise MoeError(_abi.ERR_PLAN_NOT_ROUTED, "dispatch_fp8")
        _need(x, (self.T, self.H), _BF16_LIKE, "x", dev)
        if recv8 is None:
            recv8 = torch.empty((self.recv_rows, self.H), dtype=torch.uint8, device=dev)
        if recv_scale is None:
            recv_scale = torch.empty((self.recv_rows, self.scale_blocks), dtype=torch.float32,
                                     device=dev)
        _need(recv8, (self.recv_rows, self.H), (torch.uint8,), "recv8", dev)
        _need(recv_scale, (self.recv_rows, self.scale_blocks), (torch.float32,), "recv_scale", dev)
        if self.node_dedup:
            D = self.staging_rows_max
            if staging8 is None:
                staging8 = torch.empty((D, self.H), dtype=torch.uint8, device=dev)
            if staging_scale is None:
                staging_scale = torch.empty((D, self.scale_blocks), dtype=torch.float32, device=dev)
            _need(staging8, (D, self.H), (torch.uint8,), "staging8", dev)
            _need(staging_scale, (D, self.scale_blocks), (torch.float32,), "staging_scale", dev)
        _abi.check(self._lib.moe_dispatch_fp8(self._h, _ptr(x), _ptr(recv8), _ptr(recv_scale),
                                              _ptr(staging8), _ptr(staging_scale),
                                              _stream_handle(dev, stream)), "moe_dispatch_fp8")
        return recv8, recv_scale

    # -- moe_combine_fp8
    def combine_fp8(self, y8: torch.Tensor, y_scale: torch.Tensor, topk_w: torch.Tensor,
                    out: torch.Tensor | None = None, out_dtype: torch.dtype = torch.bfloat16,
                    stream=None) -> torch.Tensor:
        dev = self.device
        if dev is None:
            raise MoeError(_abi.ERR_PLAN_NOT_ROUTED, "combine_fp8")
        _need(y8, (self.recv_rows, self.H), (torch.uint8,), "y8", dev)
        _need(y_scale, (self.recv_rows, self.scale_blocks), (torch.float32,), "y_scale", dev)
        _need(topk_w, (self.T, self.k), (torch.float32,), "topk_w", dev)
        if out_dtype not in (torch.bfloat16, torch.float32):
            raise ValueError("out_dtype must be torch.bfloat16 or torch.float32")
        if out is None:
            out = torch.empty((self.T, self.H), dtype=out_dtype, device=dev)
        _need(out, (self.T, self.H), (out_dtype,), "out", dev)
        code = _abi.OUT_F32 if out_dtype == torch.float32 else _abi.OUT_BF16
        _abi.check(self._lib.moe_combine_fp8(self._h, _ptr(y8), _ptr(y_scale), _ptr(topk_w),
                                             _ptr(out), code, _stream_handle(dev, stream)),
                   "moe_combine_fp8")
        return out

    # -- moe_plan_timing / moe_plan_timing_read
    def timing(self, capacity: int) -> None:
        """Time each kernel this plan's calls launch (up to `capacity` launches;
        0 stops).  Needs the plan's device to be current."""
        _abi.check(self._lib.moe_plan_timing(self._h, int(capacity)), "moe_plan_timing")
        self._timing_cap = int(capacity)

    def timing_read(self) -> list[tuple[str, float, float]]:
        """(kernel name, start in ms after the first launch's start, duration in ms) of
        each timed launch since the last read, in launch order."""
        cap = getattr(self, "_timing_cap", 0)
        ids = (ctypes.c_int32 * max(cap, 1))()
        start = (ctypes.c_float * max(cap, 1))()
        ms = (ctypes.c_float * max(cap, 1))()
        n = ctypes.c_int32()
        _abi.check(self._lib.moe_plan_timing_read(self._h, ids, start, ms, cap, ctypes.byref(n)),
                   "moe_plan_timing_read")
        return [(_abi.kernel_name(ids[i]), float(start[i]), float(ms[i]))
                for i in range(min(n.value, cap))]

    # -- moe_plan_read
    def read(self, item: str, stream=None) -> np.ndarray:
        nb = self.bands
        n = {"status": 1, "num_staged": 1, "counts": nb * self.E,
             "expert_offsets": nb * (self.E + 1), "rank_offsets": nb * (self.R + 1),
             "slot_of": self.T * self.k, "row_src": self.T * self.k,
             "stage_offsets": self.R + 1, "stage_of": self.T * self.k,
             "stage_src": self.staging_rows_max, "send_rows": self.R * self.R,
             "send_copies": self.R * self.R, "node_copies": self.R * self.N,
             "forwarders": self.R * self.N}[item]
        buf = np.zeros(max(n, 1), dtype=np.int32)
        dev = self.device
        if dev is None:
            raise MoeError(_abi.ERR_PLAN_NOT_ROUTED, "read")
        _abi.check(self._lib.moe_plan_read(self._h, _abi.ITEM[item],
                                           buf.ctypes.data_as(ctypes.c_void_p), buf.nbytes,
                                           _stream_handle(dev, stream)), f"moe_plan_read({item})")
        return buf[:n]

    def status(self) -> int:
        return int(self.read("status")[0])


def route_plan(topk_idx: torch.Tensor, num_experts: int, num_ranks: int, hidden: int,
               ranks_per_node: int | None = None, node_dedup: bool = False,
               load_aware_forwarders: bool = False, workspace: torch.Tensor | None = None,
               stream=None) -> Plan:
    """moe_plan_create + moe_route_plan for a [T, k] int32 routing on the GPU."""
    T, k = topk_idx.shape
    plan = Plan(T, hidden, num_experts, k, num_ranks, ranks_per_node, node_dedup,
                load_aware_forwarders)
    return plan.route(topk_idx, workspace, stream)


def dispatch(plan: Plan, x: torch.Tensor, recv=None, staging=None, stream=None):
    """moe_dispatch: returns (recv [T*k, H], staging or None)."""
    return plan.dispatch(x, recv, staging, stream)


def combine(plan: Plan, y: torch.Tensor, topk_w: torch.Tensor, out=None,
            out_dtype: torch.dtype = torch.bfloat16, stream=None) -> torch.Tensor:
    """moe_combine: returns out [T, H] (bf16 or float32)."""
    return plan.combine(y, topk_w, out, out_dtype, stream)


def dispatch_fp8(plan: Plan, x: torch.Tensor, recv8=None, recv_scale=None, staging8=None,
                 staging_scale=None, stream=None):
    """moe_dispatch_fp8: returns (codes [T*k, H] uint8, block scales [T*k, nb] float32)."""
    return plan.dispatch_fp8(x, recv8, recv_scale, staging8, staging_scale, stream)


def combine_fp8(plan: Plan, y8: torch.Tensor, y_scale: torch.Tensor, topk_w: torch.Tensor,
                out=None, out_dtype: torch.dtype = torch.bfloat16, stream=None) -> torch.Tensor:
    """moe_combine_fp8: returns out [T, H] (bf16 or float32)."""
    return plan.combine_fp8(y8, y_scale, topk_w, out, out_dtype, stream)


def combine_hier(plan: Plan, y: torch.Tensor, topk_w: torch.Tensor, partials=None, out=None,
                 out_dtype: torch.dtype = torch.bfloat16, stream=None) -> torch.Tensor:
    """moe_combine_hier: two-hop combine of a node-deduplicated plan."""
    return plan.combine_hier(y, topk_w, partials, out, out_dtype, stream)


def pipeline(plan: Plan, topk_idx: torch.Tensor, x: torch.Tensor, topk_w: torch.Tensor,
             recv=None, out=None, out_dtype: torch.dtype = torch.bfloat16, stream=None):
    """moe_pipeline: returns (recv [T*k, H], out [T, H])."""
    return plan.pipeline(topk_idx, x, topk_w, recv, out, out_dtype, stream=stream)
