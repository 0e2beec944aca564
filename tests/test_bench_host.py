"""The benchmark's host-side arithmetic (CPU): algorithmic bytes, the
one-GPU guard, the rocprofv3 summaries and the traffic lookup."""

import csv
import json
import os
import subprocess
import sys

import pytest

import bench
from combine_shuffling_amd import _abi
from workloads import gen

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("name,disp,comb", [
    ("tiny", 196_608, 196_608),
    ("olmoe", 150_994_944, 150_994_944),
    ("qwen3", 603_979_776, 603_979_776),
    ("nondiv", 939_524_096, 939_524_096),
])
def test_single_hop_bytes(name, disp, comb):
    # (T + T*k) * 2H each way: the per-workload figures of the measurement plan
    assert bench.algorithmic_bytes(gen.get(name), 0) == (disp, comb)


def test_dedup_and_variant_bytes():
    wl = gen.get("dsv3")
    T, k, row = wl.num_tokens, wl.top_k, 2 * wl.hidden
    D = 65_085
    assert bench.algorithmic_bytes(wl, D) == ((T + 2 * D + T * k) * row, (T * k + T) * row)
    # the D = 4T upper bound of the measurement plan
    assert sum(bench.algorithmic_bytes(wl, 4 * T)) == 6_106_906_624
    # hierarchical: the fp32 partials are written once and read once
    assert bench.algorithmic_bytes(wl, D, hier=True)[1] == (T * k + T) * row + 4 * D * row
    # fp8: one byte an element plus a float32 scale per 128 elements on the k rows
    row8 = wl.hidden + 4 * ((wl.hidden + 127) // 128)
    assert bench.algorithmic_bytes(gen.get("olmoe"), 0, "fp8") == \
        (4096 * 4096 + 4096 * 8 * (2048 + 64), 4096 * 8 * (2048 + 64) + 4096 * 4096)
    assert bench.algorithmic_bytes(wl, D, "fp8")[0] == T * row + (2 * D + T * k) * row8


@pytest.mark.parametrize("payload", ["bf16", "fp8"])
def test_kernel_bytes_add_up_to_the_phases(payload):
    # The per-kernel bytes of the roofline split each phase's algorithmic bytes
    # between its kernels: the two hops make up the deduplicated dispatch.
    wl, D = gen.get("dsv3"), 65_085
    kb = bench.kernel_bytes(wl, D, payload)
    sfx = "_fp8" if payload == "fp8" else ""
    disp, comb = bench.algorithmic_bytes(wl, D, payload)
    assert kb[f"stage_a{sfx}_kernel"] + kb[f"stage_b{sfx}_kernel"] == disp
    assert kb[f"combine{sfx}_kernel"] == comb
    one = gen.get("nondiv")
    kb1 = bench.kernel_bytes(one, 0, payload)
    d1, c1 = bench.algorithmic_bytes(one, 0, payload)
    assert kb1[f"gather{sfx}_kernel"] == kb1[f"gather{sfx}_scan_kernel"] == d1
    assert kb1[f"combine{sfx}_kernel"] == c1
    # the fused launches of the chunked calls share out the same bytes
    tc, dc = [2048] * 8, [8136] * 7 + [D - 7 * 8136]
    kc = bench.kernel_bytes(wl, D, payload, (tc, dc), (tc, dc))
    assert kc[f"stage_a{sfx}_kernel"] + kc[f"stage_ab{sfx}_kernel"] + kc[f"stage_b{sfx}_kernel"] == disp
    hd, hc = bench.algorithmic_bytes(wl, D, hier=True)
    assert kc["combine_part_kernel"] + kc["combine_pn_kernel"] + kc["combine_nodes_kernel"] == hc
    assert kb["combine_part_kernel"] + kb["combine_nodes_kernel"] == hc
    assert kb1["pipeline_kernel"] == sum(bench.algorithmic_bytes(one, 0))


def test_default_is_the_largest_workload():
    # The headline is the DeepSeek-V3-like shuffle (the largest configuration);
    # the other large workloads are measured in the same run.
    a = bench.parse([])
    assert a.workload == "dsv3" and a.payload == "bf16"
    assert set(a.configs.split(",")) == {"olmoe", "qwen3", "nondiv"}


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def _write_csv(path, rows, fields):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=fields)
        w.writeheader()
        w.writerows(rows)


def test_pmc_summary_scales_by_the_copy_kernel(tmp_path):
    fields = ["Kernel_Name", "Counter_Name", "Counter_Value"]
    kern = "void moe::(anonymous namespace)::combine_kernel<8, 1, false>(moe::Dims)"
    copy = "void at::native::vectorized_elementwise_kernel<8>(int)"
    # FETCH_SIZE reads half of what moved (as measured on gfx950), WRITE_SIZE all of it
    _write_csv(tmp_path / "f.csv", [dict(Kernel_Name=kern, Counter_Name="FETCH_SIZE",
                                         Counter_Value=v) for v in (100.0, 102.0)], fields)
    _write_csv(tmp_path / "w.csv", [dict(Kernel_Name=kern, Counter_Name="WRITE_SIZE",
                                         Counter_Value=v) for v in (50.0, 50.0)], fields)
    _write_csv(tmp_path / "cf.csv", [dict(Kernel_Name=copy, Counter_Name="FETCH_SIZE",
                                          Counter_Value=512.0)] * 5, fields)
    _write_csv(tmp_path / "cw.csv", [dict(Kernel_Name=copy, Counter_Name="WRITE_SIZE",
                                          Counter_Value=1024.0)] * 5, fields)
    out = tmp_path / "s.txt"
    bench.summarize_pmc(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), str(tmp_path / "cf.csv"),
                        str(tmp_path / "cw.csv"), str(out), 1, "cmd")
    text = "".join(ln for ln in open(out) if not ln.startswith("#"))
    s = json.loads(text)
    assert s["fetch_factor"] == 2.0 and s["write_factor"] == 1.0
    k = s["kernels"]["combine_kernel<8, 1, false>"]
    assert k["dispatches"] == 2
    assert k["traffic_bytes"] == int((101.0 * 2 + 50.0) * 1024)
    assert s["source_hashes"] == {"move.hip": bench.kernel_source_hash("move.hip")}
    assert s["command"] == "cmd"


def test_trace_summary(tmp_path):
    fields = ["Name", "Calls", "AverageNs", "MinNs", "MaxNs"]
    _write_csv(tmp_path / "t.csv", [dict(Name="void moe::gather_kernel<8, 1>()", Calls=110,
                                         AverageNs=26550.0, MinNs=25000.0, MaxNs=30000.0)], fields)
    out = tmp_path / "t.txt"
    bench.summarize_trace(str(tmp_path / "t.csv"), str(out), "cmd")
    lines = open(out).read().splitlines()
    assert lines[1] == "# command: cmd"
    assert lines[3].split()[-4:] == ["110", "26.55", "25.00", "30.00"]


def test_traffic_lookup_needs_current_sources(tmp_path, monkeypatch):
    summary = {"source_hashes": {"move.hip": bench.kernel_source_hash("move.hip"),
                                 "pipeline.hip": "0" * 16},  # changed since
               "kernels": {"gather_kernel<8, 1>": {"traffic_bytes": 123},
                           "combine_kernel<8, 1, false>": {"traffic_bytes": 456},
                           "pipeline_kernel<8, false>": {"traffic_bytes": 789}}}
    (tmp_path / "hbm_traffic_w.txt").write_text("# header\n" + json.dumps(summary))
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    assert bench.recorded_traffic("w", "gather_kernel") == ("gather_kernel<8, 1>", 123)
    assert bench.recorded_traffic("w", "gather_scan_kernel") == (None, None)
    assert bench.recorded_traffic("w", "combine_kernel") == ("combine_kernel<8, 1, false>", 456)
    assert bench.recorded_traffic("w", "stage_a_kernel") == (None, None)
    assert bench.recorded_traffic("missing", "gather_kernel") == (None, None)
    assert bench.recorded_traffic("w", "pipeline_kernel") == (None, None)
    summary["source_hashes"]["move.hip"] = "0" * 16   # the kernels changed since
    (tmp_path / "hbm_traffic_w.txt").write_text(json.dumps(summary))
    assert bench.recorded_traffic("w", "gather_kernel") == (None, None)


def test_kernel_units():
    assert bench.kernel_unit("void moe::(anonymous namespace)::pipeline_kernel<8, false>(m") \
        == "pipeline.hip"
    assert bench.kernel_unit("counters_clear_kernel") == "pipeline.hip"
    assert bench.kernel_unit("route_count_kernel<8>") == "route_plan.hip"
    assert bench.kernel_unit("stage_ab_kernel<8>") == "move.hip"
    # defined in a shared header, launched by move.hip
    assert bench.kernel_unit("combine_kernel<8, 1, false>") == "move.hip"
    assert bench.kernel_unit("gather_kernel<8, 1>") == "move.hip"
    with pytest.raises(ValueError):
        bench.kernel_unit("no_such_kernel")
    hashes = {u: bench.kernel_source_hash(u) for u in bench.KERNEL_UNITS}
    assert len(set(hashes.values())) == 3


def test_every_library_kernel_has_one_unit():
    """Each kernel the library can time (moe_kernel_name) maps to exactly one
    translation unit, so its traffic summary is checked against the right sources."""
    names = [_abi.kernel_name(i) for i in range(_abi.KERNEL_COUNT)]
    assert "?" not in names and len(set(names)) == _abi.KERNEL_COUNT
    for n in names:
        bench.kernel_unit(n)

