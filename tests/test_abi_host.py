"""The C ABI on the host (CPU, no GPU needed): the library loads, exports every
function include/moe_shuffle.h declares, and rejects bad configurations before
anything is launched."""

import ctypes
import os
import re

import numpy as np
import pytest

from combine_shuffling_amd import _abi

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include",
                      "moe_shuffle.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    lib = _abi.lib()
    names = declared_functions()
    assert set(names) == set(_abi.EXPORTS), names
    for n in names:
        assert hasattr(lib, n), n


def make(T=128, H=256, E=8, k=2, R=2, G=None, flags=0, band=0):
    cfg = _abi.MoeConfig(T, H, E, k, R, R if G is None else G, flags, band)
    h = ctypes.c_void_p()
    st = _abi.lib().moe_plan_create(ctypes.byref(cfg), ctypes.byref(h))
    return st, h


@pytest.mark.parametrize("kw,want", [
    (dict(), _abi.OK),
    (dict(T=0), _abi.OK),
    (dict(T=-1), _abi.ERR_INVALID_ARGUMENT),
    (dict(H=0), _abi.ERR_INVALID_ARGUMENT),
    (dict(H=12), _abi.ERR_INVALID_ARGUMENT),          # row not a whole number of 16-byte chunks
    (dict(E=0), _abi.ERR_INVALID_ARGUMENT),
    (dict(k=0), _abi.ERR_INVALID_ARGUMENT),
    (dict(k=9), _abi.ERR_INVALID_ARGUMENT),           # k > E
    (dict(E=2, R=8), _abi.ERR_EXPERTS_LT_RANKS),      # zero-expert ranks
    (dict(E=8, R=3, G=2), _abi.ERR_INVALID_ARGUMENT),  # G does not divide R
    (dict(E=2048, k=2), _abi.ERR_UNSUPPORTED),
    (dict(E=64, k=17, R=4), _abi.ERR_UNSUPPORTED),
    (dict(flags=_abi.FLAG_NODE_DEDUP), _abi.ERR_INVALID_ARGUMENT),  # one node: nothing to dedup
    (dict(R=2, G=1, flags=_abi.FLAG_NODE_DEDUP), _abi.OK),
    (dict(flags=4), _abi.ERR_INVALID_ARGUMENT),
    (dict(R=2, G=1, flags=_abi.FLAG_LOAD_AWARE_FORWARDERS), _abi.ERR_INVALID_ARGUMENT),  # needs dedup
    (dict(R=2, G=1, flags=_abi.FLAG_NODE_DEDUP | _abi.FLAG_LOAD_AWARE_FORWARDERS), _abi.OK),
    (dict(E=1024, R=1024, G=1, flags=_abi.FLAG_NODE_DEDUP | _abi.FLAG_LOAD_AWARE_FORWARDERS),
     _abi.ERR_UNSUPPORTED),                            # R*N past the key space
    (dict(T=1 << 28, k=8), _abi.ERR_UNSUPPORTED),     # T*k past 32-bit row indices
    (dict(T=(2 ** 31 - 4096) // 8, k=8), _abi.ERR_UNSUPPORTED),  # inside the 4096 margin
    (dict(T=(2 ** 31 - 4097) // 8 - 1, H=8, k=8, E=16), _abi.OK),  # just below it
    (dict(T=4096, band=512), _abi.OK),
    (dict(T=4096, band=100), _abi.ERR_INVALID_ARGUMENT),   # not a multiple of 256
    (dict(T=4096, band=-256), _abi.ERR_INVALID_ARGUMENT),
    (dict(T=4096, band=8192), _abi.OK),                   # one band
    (dict(T=4096, E=1024, k=2, band=4096 - 256), _abi.ERR_UNSUPPORTED),  # 15 tiles x 1024 > LDS
    (dict(T=256 * 193, band=256), _abi.ERR_UNSUPPORTED),  # more than 192 bands
    (dict(T=4096, R=4, G=2, flags=_abi.FLAG_NODE_DEDUP, band=512), _abi.ERR_UNSUPPORTED),
])
def test_plan_create_status(kw, want):
    st, h = make(**kw)
    assert st == want, _abi.status_str(st)
    if st == _abi.OK:
        _abi.lib().moe_plan_destroy(h)


def test_plan_sizes():
    L = _abi.lib()
    st, h = make(T=16384, H=7168, E=256, k=8, R=64, G=8, flags=_abi.FLAG_NODE_DEDUP)
    assert st == _abi.OK
    assert L.moe_plan_recv_rows(h) == 16384 * 8
    assert L.moe_plan_staging_rows_max(h) == 16384 * 8   # min(k, N) = 8
    ws = L.moe_plan_workspace_bytes(h)
    assert ws % 256 == 0 and ws >= 4 * (3 * 16384 * 8)
    L.moe_plan_destroy(h)
    st, h = make(T=4096, H=2048, E=64, k=8, R=4)
    assert L.moe_plan_staging_rows_max(h) == 0
    L.moe_plan_destroy(h)
    L.moe_plan_destroy(None)


def test_workloads_fit_the_static_workspace():
    # Every workload's plan fits the static workspace of moe_route_plan_static
    # (the DeepSeek-V3-like one also with load-aware forwarders), and the
    # load-aware layout holds, besides the wider [tiles x (owner, node)] count
    # and base matrices, the per-(tile, node) staging sums.
    from workloads import gen

    L = _abi.lib()
    sizes = {}
    for name in ("tiny", "olmoe", "qwen3", "dsv3", "nondiv"):
        wl = gen.get(name)
        flags = _abi.FLAG_NODE_DEDUP if wl.node_dedup else 0
        st, h = make(wl.num_tokens, wl.hidden, wl.num_experts, wl.top_k, wl.num_ranks,
                     wl.ranks_per_node, flags)
        assert st == _abi.OK, name
        sizes[name] = L.moe_plan_workspace_bytes(h)
        L.moe_plan_destroy(h)
        assert 0 < sizes[name] <= _abi.STATIC_WORKSPACE_BYTES, name
    wl = gen.get("dsv3")
    st, h = make(wl.num_tokens, wl.hidden, wl.num_experts, wl.top_k, wl.num_ranks,
                 wl.ranks_per_node, _abi.FLAG_NODE_DEDUP | _abi.FLAG_LOAD_AWARE_FORWARDERS)
    assert st == _abi.OK
    la = L.moe_plan_workspace_bytes(h)
    L.moe_plan_destroy(h)
    assert la <= _abi.STATIC_WORKSPACE_BYTES
    R, N, tiles = wl.num_ranks, wl.num_ranks // wl.ranks_per_node, 64
    # arrays are 256-byte aligned; the static plan keeps one slot of 256 bytes
    # in place of the per-node sums
    assert la - sizes["dsv3"] == 4 * (2 * tiles * (R * N - R) + tiles * N) - 256


def test_calls_before_route_are_refused():
    L = _abi.lib()
    st, h = make()
    buf = np.zeros(16, dtype=np.int32)
    vp = ctypes.c_void_p
    assert L.moe_dispatch(h, vp(16), vp(16), None, None) == _abi.ERR_PLAN_NOT_ROUTED
    assert L.moe_combine(h, vp(16), vp(16), vp(16), 0, None) == _abi.ERR_PLAN_NOT_ROUTED
    assert L.moe_plan_read(h, 0, buf.ctypes.data_as(vp), buf.nbytes, None) == \
        _abi.ERR_PLAN_NOT_ROUTED
    # null / misaligned workspace is refused before any launch
    assert L.moe_route_plan(h, vp(256), None, None) == _abi.ERR_INVALID_ARGUMENT
    assert L.moe_route_plan(h, vp(256), vp(1024 + 8), None) == _abi.ERR_INVALID_ARGUMENT
    L.moe_plan_destroy(h)


def test_expert_partition_matches_printed_and_oracle():
    import oracle
    from combine_shuffling_amd import expert_partition, MoeError

    for E, R in [(256, 7), (100, 7), (384, 5), (384, 6), (384, 7), (8, 2), (1, 1), (1024, 1000)]:
        assert expert_partition(E, R) == oracle.expert_partition(E, R).tolist()
    assert np.diff(expert_partition(256, 7)).tolist() == [37, 37, 37, 37, 36, 36, 36]
    assert np.diff(expert_partition(100, 7)).tolist() == [15, 15, 14, 14, 14, 14, 14]
    with pytest.raises(MoeError) as ei:
        expert_partition(2, 8)
    assert ei.value.status == _abi.ERR_EXPERTS_LT_RANKS
    with pytest.raises(MoeError):
        expert_partition(0, 1)


def test_band_counts():
    L = _abi.lib()
    for T, band, nb in [(4096, 512, 8), (4000, 512, 8), (4096, 0, 1), (4096, 8192, 1), (0, 256, 1),
                        (257, 256, 2)]:
        st, h = make(T=T, band=band)
        assert st == _abi.OK
        assert L.moe_plan_bands(h) == nb, (T, band)
        L.moe_plan_destroy(h)


def test_pipeline_refused_on_host():
    L = _abi.lib()
    vp = ctypes.c_void_p
    st, h = make(T=64)
    assert L.moe_pipeline(h, vp(16), None, vp(16), vp(16), vp(16), vp(16), 0, None) == \
        _abi.ERR_INVALID_ARGUMENT                       # no workspace
    assert L.moe_pipeline(h, vp(16), vp(1024), vp(16), vp(16), vp(16), vp(16), 7, None) == \
        _abi.ERR_INVALID_ARGUMENT                       # bad out dtype
    assert L.moe_pipeline(h, vp(18), vp(1024), vp(16), vp(16), vp(16), vp(16), 0, None) == \
        _abi.ERR_INVALID_ARGUMENT                       # misaligned routing
    assert L.moe_pipeline(h, vp(16), vp(1024), vp(16), vp(16 + 64), vp(16), vp(16), 0, None) == \
        _abi.ERR_INVALID_ARGUMENT                       # recv not 128-byte aligned
    L.moe_plan_destroy(h)
    st, h = make(T=64, H=200)                           # rows not whole 128-byte lines
    assert L.moe_pipeline(h, vp(16), vp(1024), vp(16), vp(16), vp(16), vp(16), 0, None) == \
        _abi.ERR_UNSUPPORTED
    L.moe_plan_destroy(h)
    st, h = make(T=64, R=2, G=1, flags=_abi.FLAG_NODE_DEDUP)
    assert L.moe_pipeline(h, vp(16), vp(1024), vp(16), vp(16), vp(16), vp(16), 0, None) == \
        _abi.ERR_UNSUPPORTED
    L.moe_plan_destroy(h)


def test_status_strings():
    for s in range(8):
        assert _abi.status_str(s)
    assert "unknown" in _abi.status_str(99)


def test_fp8_entry_points_on_host():
    L = _abi.lib()
    st, h = make(T=64, H=200)
    assert L.moe_plan_scale_blocks(h) == 2          # ceil(200 / 128)
    vp = ctypes.c_void_p
    assert L.moe_dispatch_fp8(h, vp(16), vp(16), vp(16), None, None, None) == _abi.ERR_PLAN_NOT_ROUTED
    assert L.moe_combine_fp8(h, vp(16), vp(16), vp(16), vp(16), 0, None) == _abi.ERR_PLAN_NOT_ROUTED
    L.moe_plan_destroy(h)


def test_kernel_names_are_the_kernels_symbols():
    # Every moe_kernel id names a __global__ function of the sources, as a
    # profiler lists it; ids outside the enum give "?".
    csrc = os.path.join(os.path.dirname(HEADER), "..", "combine_shuffling_amd", "csrc")
    text = "".join(open(os.path.join(csrc, f)).read() for f in os.listdir(csrc)
                   if f.endswith((".hip", ".h")))
    kernels = set(re.findall(r"void\s+(\w+_kernel)\s*\(", text))
    names = [_abi.kernel_name(i) for i in range(_abi.KERNEL_COUNT)]
    assert len(set(names)) == _abi.KERNEL_COUNT
    assert set(names) <= kernels, set(names) - kernels
    assert _abi.kernel_name(_abi.KERNEL_COUNT) == "?" and _abi.kernel_name(-1) == "?"


def test_timing_host_errors():
    L = _abi.lib()
    st, h = make()
    assert st == _abi.OK
    n = ctypes.c_int32()
    ids = (ctypes.c_int32 * 1)()
    ms = (ctypes.c_float * 1)()
    st = (ctypes.c_float * 1)()
    assert L.moe_plan_timing(None, 4) == _abi.ERR_INVALID_ARGUMENT
    assert L.moe_plan_timing(h, -1) == _abi.ERR_INVALID_ARGUMENT
    assert L.moe_plan_timing(h, 0) == _abi.OK                     # off: no HIP call
    assert L.moe_plan_timing_read(h, ids, st, ms, 1, ctypes.byref(n)) == _abi.ERR_INVALID_ARGUMENT
    L.moe_plan_destroy(h)


@pytest.mark.parametrize("T,H,k,R,G,want", [
    (16384, 7168, 8, 64, 8, 2048),   # DeepSeek-V3-like: 8 chunks
    (2500, 7168, 8, 16, 2, 1250),    # 2 chunks
    (4999, 7168, 8, 8, 1, 1667),     # 3 chunks, the last ragged
    (300, 64, 4, 8, 2, 300),         # one chunk
    (4096, 2048, 8, 4, 4, 4096),     # single hop: the whole batch
])
def test_dispatch_chunk_tokens(T, H, k, R, G, want):
    import combine_shuffling_amd as cs

    p = cs.Plan(T, H, 64, k, R, G, R // G > 1)
    assert p.chunk_tokens["dispatch"] == want


def test_chunk_tokens_of_the_fp8_dispatch_and_hierarchical_combine():
    import combine_shuffling_amd as cs

    p = cs.Plan(16384, 7168, 256, 8, 64, 8, True)
    # fp8: 8 rows of 7168 codes + 56 scales a token -> 5 chunks; hierarchical
    # combine: 8 fp32 partial rows a token, at most 448 MiB a chunk -> 8 chunks
    assert p.chunk_tokens == {"dispatch": 2048, "dispatch_fp8": 3277, "combine_hier": 2048}
    one = cs.Plan(4096, 2048, 64, 8, 4)
    assert set(one.chunk_tokens.values()) == {4096}
