"""ctypes declarations of the C ABI in include/moe_shuffle.h.

Loads the in-tree libmoeshuffle.so and fails loudly when it is missing: there
is no fallback of any kind.
"""

from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoeshuffle.so")

# moe_status
OK = 0
ERR_INVALID_ARGUMENT = 1
ERR_EXPERTS_LT_RANKS = 2
ERR_BAD_ROUTING = 3
ERR_PLAN_NOT_ROUTED = 4
ERR_HIP = 5
ERR_UNSUPPORTED = 6
ERR_PIPELINE_STALL = 7
ERR_STATIC_WORKSPACE = 8
STATIC_WORKSPACE_BYTES = 32 << 20

FLAG_NODE_DEDUP = 1
FLAG_LOAD_AWARE_FORWARDERS = 2
MAX_EXPERTS = 1024
MAX_TOPK = 16

OUT_BF16 = 0
OUT_F32 = 1

# moe_item
ITEM = dict(status=0, counts=1, expert_offsets=2, rank_offsets=3, slot_of=4, row_src=5,
            num_staged=6, stage_offsets=7, stage_of=8, stage_src=9, send_rows=10,
            send_copies=11, node_copies=12, forwarders=13)


class MoeConfig(ctypes.Structure):
    _fields_ = [
        ("num_tokens", ctypes.c_int64),
        ("hidden", ctypes.c_int32),
        ("num_experts", ctypes.c_int32),
        ("top_k", ctypes.c_int32),
        ("num_ranks", ctypes.c_int32),
        ("ranks_per_node", ctypes.c_int32),
        ("flags", ctypes.c_uint32),
        ("band_tokens", ctypes.c_int32),
    ]


EXPORTS = (
    "moe_expert_partition", "moe_plan_create", "moe_plan_destroy", "moe_plan_workspace_bytes",
    "moe_plan_recv_rows", "moe_plan_staging_rows_max", "moe_route_plan", "moe_dispatch",
    "moe_combine", "moe_plan_read", "moe_status_str", "moe_plan_scale_blocks",
    "moe_dispatch_fp8", "moe_combine_fp8", "moe_combine_hier", "moe_plan_bands", "moe_pipeline",
    "moe_kernel_name", "moe_plan_timing", "moe_plan_timing_read", "moe_route_plan_static",
    "moe_plan_chunk_tokens",
)

KERNEL_COUNT = 22


class MoeError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_str(status)} (status {status})")


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python -m combine_shuffling_amd.build` "
            "(hipcc, gfx950). There is no fallback path.")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    L.moe_expert_partition.argtypes = [i32, i32, ctypes.POINTER(i32)]
    L.moe_expert_partition.restype = i32
    L.moe_plan_create.argtypes = [ctypes.POINTER(MoeConfig), ctypes.POINTER(vp)]
    L.moe_plan_create.restype = i32
    L.moe_plan_destroy.argtypes = [vp]
    L.moe_plan_destroy.restype = None
    L.moe_plan_workspace_bytes.argtypes = [vp]
    L.moe_plan_workspace_bytes.restype = sz
    L.moe_plan_recv_rows.argtypes = [vp]
    L.moe_plan_recv_rows.restype = i64
    L.moe_plan_staging_rows_max.argtypes = [vp]
    L.moe_plan_staging_rows_max.restype = i64
    L.moe_route_plan.argtypes = [vp, vp, vp, vp]
    L.moe_route_plan.restype = i32
    L.moe_dispatch.argtypes = [vp, vp, vp, vp, vp]
    L.moe_dispatch.restype = i32
    L.moe_combine.argtypes = [vp, vp, vp, vp, i32, vp]
    L.moe_combine.restype = i32
    L.moe_plan_read.argtypes = [vp, i32, vp, sz, vp]
    L.moe_plan_read.restype = i32
    L.moe_plan_scale_blocks.argtypes = [vp]
    L.moe_plan_scale_blocks.restype = i64
    L.moe_dispatch_fp8.argtypes = [vp, vp, vp, vp, vp, vp, vp]
    L.moe_dispatch_fp8.restype = i32
    L.moe_combine_fp8.argtypes = [vp, vp, vp, vp, vp, i32, vp]
    L.moe_combine_fp8.restype = i32
    L.moe_combine_hier.argtypes = [vp, vp, vp, vp, vp, i32, vp]
    L.moe_combine_hier.restype = i32
    L.moe_plan_chunk_tokens.argtypes = [vp, i32]
    L.moe_plan_chunk_tokens.restype = i64
    L.moe_plan_bands.argtypes = [vp]
    L.moe_plan_bands.restype = i64
    L.moe_pipeline.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, vp]
    L.moe_pipeline.restype = i32
    L.moe_route_plan_static.argtypes = [vp, vp, vp]
    L.moe_route_plan_static.restype = i32
    L.moe_kernel_name.argtypes = [i32]
    L.moe_kernel_name.restype = ctypes.c_char_p
    L.moe_plan_timing.argtypes = [vp, i32]
    L.moe_plan_timing.restype = i32
    L.moe_plan_timing_read.argtypes = [vp, ctypes.POINTER(i32), ctypes.POINTER(ctypes.c_float),
                                       ctypes.POINTER(ctypes.c_float), i32, ctypes.POINTER(i32)]
    L.moe_plan_timing_read.restype = i32
    L.moe_status_str.argtypes = [i32]
    L.moe_status_str.restype = ctypes.c_char_p
    _lib = L
    return L


def kernel_name(kernel: int) -> str:
    return lib().moe_kernel_name(kernel).decode()


def status_str(status: int) -> str:
    return lib().moe_status_str(status).decode()


def check(status: int, what: str) -> None:
    if status != OK:
        raise MoeError(status, what)
