"""bench.py's host-side bookkeeping, without a GPU: the algorithmic byte count
behind roofline.achieved, the number of launches per captured graph, and the
rule that HBM counters are reported only for the sources they were taken on."""
import json
import os
import sys

import pytest

from conftest import ROOT

sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_algorithmic_bytes_of_the_4096_square_layer():
    # Per 32 weights: 96 code bits + one scale byte = 13 bytes (3.25 bits per
    # weight); 8 codebook bytes per row; bf16 activations; fp32 outputs.
    payload = 4096 * 4096 // 32 * 13
    assert payload == 6_815_744
    assert bench.algorithmic_bytes(4096, 4096, 1) == payload + 8 * 4096 + 2 * 4096 + 4 * 4096 == 6_873_088
    assert bench.algorithmic_bytes(4096, 4096, 8) == payload + 8 * 4096 + 8 * (2 * 4096 + 4 * 4096)
    # the vocabulary projection at 64 tokens
    assert bench.algorithmic_bytes(151936, 4096, 64) == 252_821_504 + 1_215_488 + 524_288 + 38_895_616


@pytest.mark.parametrize("copies", [1, 3, 6, 63, 64, 65, 79, 1261])
def test_graph_holds_the_fewest_whole_passes_reaching_the_launch_floor(copies):
    c = bench.cycles_for(copies)
    assert c >= 1
    assert c * copies >= bench.GRAPH_LAUNCHES
    assert c == 1 or (c - 1) * copies < bench.GRAPH_LAUNCHES


def _write_traffic(tmp_path, source_hash, kernels):
    p = tmp_path / "traffic.json"
    p.write_text(json.dumps({"source_hash": source_hash, "fetch_scale": 2.0, "write_scale": 1.0,
                             "kernels": kernels}))
    return str(p)


KERNELS = {
    "splitk_kernel<16, 1, true, 1>": {"read_bytes": 7_029_704, "write_bytes": 16_384, "dispatches": 633},
    "splitk_kernel<16, 1, false, 1>": {"read_bytes": 7_053_214, "write_bytes": 16_384, "dispatches": 1344},
    "splitk_kernel<4, 1, false, 1>": {"read_bytes": 5, "write_bytes": 5, "dispatches": 99999},
    "linear_kernel<1, 1, 8, 1, 0, false, 3>": {"read_bytes": 1, "write_bytes": 1, "dispatches": 99999},
    "linear_kernel<1, 1, 8, 0, 0, false, 2>": {"read_bytes": 2, "write_bytes": 2, "dispatches": 99999},
    "pack_kernel": {"read_bytes": 3, "write_bytes": 3, "dispatches": 1},
}


def test_traffic_is_read_for_the_matching_sources(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "TRAFFIC_FILE", _write_traffic(tmp_path, bench.source_hash(), KERNELS))
    name, v = bench.read_traffic(True)
    assert name == "splitk_kernel<16, 1, true, 1>" and v["read_bytes"] == 7_029_704
    # the matrix-core instance; other shapes' instances, expert passes and 2-bit kernels are never taken for it
    name, v = bench.read_traffic(False)
    assert name == "splitk_kernel<16, 1, false, 1>" and v["read_bytes"] == 7_053_214


def test_traffic_from_other_sources_is_not_reported(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "TRAFFIC_FILE", _write_traffic(tmp_path, "0" * 16, KERNELS))
    assert bench.read_traffic(True) == ("splitk_kernel (vector-ALU, M=1)", None)
    monkeypatch.setattr(bench, "TRAFFIC_FILE", os.path.join(str(tmp_path), "missing.json"))
    assert bench.read_traffic(False) == ("splitk_kernel (matrix-core, M=1)", None)



def test_union_traffic_is_twice_the_expert_pass_average(tmp_path, monkeypatch):
    # Gate/up and down are one kernel instance (grouping 1), one dispatch each per round.
    k = {n: v for n, v in KERNELS.items() if ", 1, 0, false, 3>" not in n}
    k["linear_kernel<1, 1, 4, 1, 0, false, 3>"] = {"read_bytes": 41_000_000, "write_bytes": 10, "dispatches": 40}
    monkeypatch.setattr(bench, "MOE_TRAFFIC_FILE", _write_traffic(tmp_path, bench.source_hash(), k))
    t = bench.moe_traffic()
    assert t["read_bytes_per_round"] == 82_000_000 and t["kernel"] == "linear_kernel<1, 1, 4, 1, 0, false, 3>"
    monkeypatch.setattr(bench, "MOE_TRAFFIC_FILE", _write_traffic(tmp_path, "1" * 16, k))
    assert bench.moe_traffic() is None


def _counter_csv(path, counter, rows):
    with open(path, "w") as f:
        f.write("Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value\n")
        for i, (kern, val) in enumerate(rows):
            f.write(f'{i},"{kern}",{counter},{val}\n')
    return str(path)


def test_counter_files_are_scaled_by_the_calibration_copy(tmp_path):
    import bench_traffic
    kern = "void q3::(anonymous namespace)::linear_kernel<1, 1, 4, 0, 0, true, 3>(q3::KArgs)"
    copy = "__amd_rocclr_copyBuffer"
    # The counter sees half of the copy's 256 MiB read and all of its write.
    f = _counter_csv(tmp_path / "f.csv", "FETCH_SIZE", [(copy, 128 * 1024), (copy, 10), (kern, 3000), (kern, 3200)])
    w = _counter_csv(tmp_path / "w.csv", "WRITE_SIZE", [(copy, 256 * 1024), (kern, 16)])
    out = bench_traffic.merge([(f, w)])
    v = out["kernels"]["linear_kernel<1, 1, 4, 0, 0, true, 3>"]
    assert v["read_bytes"] == 2 * 3100 * 1024 and v["write_bytes"] == 16 * 1024 and v["dispatches"] == 2
    assert out["source_hash"] == bench.source_hash()
