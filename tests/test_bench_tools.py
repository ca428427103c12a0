"""Host logic of bench.py's profile tooling: the rocprofv3 CSV condensers and
the counter-to-bytes arithmetic of the traffic record (no GPU)."""
import csv
import json
import os
import sys

import pytest

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import bench  # noqa: E402


def _write_pmc(d, rows):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "x_counter_collection.csv"), "w", newline="") as fh:
        w = csv.writer(fh)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value"])
        for r in rows:
            w.writerow(r)


def test_pmc_summary_sums_instances_and_filters(tmp_path):
    _write_pmc(str(tmp_path / "p"), [
        (7, "void moe::gemm_fp8_kernel<0, 160>(moe::GemmArgs)", 100, "FETCH_SIZE", 10.0),
        (7, "void moe::gemm_fp8_kernel<0, 160>(moe::GemmArgs)", 100, "FETCH_SIZE", 5.0),
        (8, "at::elementwise_kernel", 50, "FETCH_SIZE", 99.0),
    ])
    out = str(tmp_path / "s.txt")
    assert bench.pmc_summary(str(tmp_path / "p"), out) == 1
    rows = bench._read_pmc_summary(out)
    assert rows == [(7, "void moe::gemm_fp8_kernel<0, 160>(moe::GemmArgs)", "100", {"FETCH_SIZE": 15.0})]
    assert bench.pmc_summary(str(tmp_path / "p"), out, "elementwise") == 1


def test_record_traffic_scales_by_the_copy_and_picks_the_launch(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILE_TRAFFIC", str(tmp_path / "traffic.json"))
    k = "void moe::gemm_bf16_kernel<0, 256, 2, 2>(moe::GemmArgs)"
    # two calls, each with two launches of the kernel (the second is the one asked for)
    _write_pmc(str(tmp_path / "f"), [(1, k, 1, "FETCH_SIZE", 100.0), (2, k, 1, "FETCH_SIZE", 300.0),
                                     (3, k, 1, "FETCH_SIZE", 100.0), (4, k, 1, "FETCH_SIZE", 500.0)])
    _write_pmc(str(tmp_path / "w"), [(1, k, 1, "WRITE_SIZE", 1.0), (2, k, 1, "WRITE_SIZE", 20.0),
                                     (3, k, 1, "WRITE_SIZE", 1.0), (4, k, 1, "WRITE_SIZE", 40.0)])
    # a 1 MiB copy whose counters read 512 KiB fetched and 1024 KiB written
    _write_pmc(str(tmp_path / "cf"), [(1, "at::copy_kernel", 1, "FETCH_SIZE", 512.0)])
    _write_pmc(str(tmp_path / "cw"), [(1, "at::copy_kernel", 1, "WRITE_SIZE", 1024.0)])
    paths = {}
    for n, pat in (("f", "moe::"), ("w", "moe::"), ("cf", "copy"), ("cw", "copy")):
        paths[n] = str(tmp_path / (n + ".txt"))
        bench.pmc_summary(str(tmp_path / n), paths[n], pat)
    ent = bench.record_traffic("wl", "gateup[x]", "gemm_bf16_kernel<0, 256,#1/2", paths["f"], paths["w"], paths["cf"],
                               paths["cw"], 1 << 20)
    # fetch: mean(300, 500) KiB x 2, write: mean(20, 40) KiB x 1
    assert ent["fetch_bytes"] == pytest.approx(800.0 * 1024)
    assert ent["write_bytes"] == pytest.approx(30.0 * 1024)
    assert ent["bytes"] == pytest.approx(830.0 * 1024)
    assert ent["symbol"] == "gemm_bf16_kernel<0, 256,"
    stored = json.load(open(tmp_path / "traffic.json"))
    assert stored["wl"]["gateup[x]"]["bytes"] == ent["bytes"]
    assert bench.stored_traffic("wl", "gateup[x]") == ent["bytes"]
    # a different kernel's stored hash does not validate this one
    stored["wl"]["gateup[x]"]["source_hash"] = "0" * 16
    json.dump(stored, open(tmp_path / "traffic.json", "w"))
    assert bench.stored_traffic("wl", "gateup[x]") is None
    with pytest.raises(SystemExit):
        bench.record_traffic("wl", "k", "gemm_bf16_kernel<0, 256,#0/3", paths["f"], paths["w"], paths["cf"],
                             paths["cw"], 1 << 20)


def test_kernel_source_hash_follows_the_kernels_own_units():
    # the fp8 and bf16 GEMMs live in different units: their hashes differ, and
    # each is stable
    a = bench._kernel_source_hash("gemm_fp8_kernel<0, 160>")
    b = bench._kernel_source_hash("gemm_bf16_kernel<0, 128, 2, 2>")
    assert a != b and a == bench._kernel_source_hash("gemm_fp8_kernel<2, 160>")


def test_short_kernel_names():
    assert bench._short_kernel("void moe::(anonymous namespace)::norm_route_kernel<false, true, 40>"
                               "(moe::(anonymous namespace)::NormRouteArgs)") == "norm_route_kernel<false, true, 40>"
    assert bench._short_kernel("moe::router_finish_kernel(moe::RouterArgs, int, float const*)") == "router_finish_kernel"
    assert bench._kernel_role("gemm_fp8_kernel<2, 160>").startswith("routed down")


def test_trace_summary_splits_calls(tmp_path):
    d = tmp_path / "t"
    d.mkdir()
    names = ["void moe::scan_kernel(int)", "void moe::gemm_fp8_kernel<0, 160>(moe::GemmArgs)",
             "void moe::gemm_fp8_tall_kernel<0>(moe::GemmArgs)"]
    with open(d / "k_kernel_trace.csv", "w", newline="") as fh:
        w = csv.writer(fh)
        w.writerow(["Queue_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        t = 0
        for c in range(6):   # warmup 1, steps 2: 2 + 4 calls
            for i, n in enumerate(names):
                w.writerow([2 if i == 2 else 1, n, t + 1000 * c, t + 1000 * c + 100 * (c + 1)])
                t += 10
            w.writerow([1, "at::fill_kernel", t, t + 1])
    with open(d / "k_kernel_stats.csv", "w", newline="") as fh:
        w = csv.writer(fh)
        w.writerow(["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs", "MaxNs", "StdDev"])
        for n in names:
            w.writerow([n, 6, 600, 100, 33, 100, 100, 0])
    out = tmp_path / "o.md"
    assert bench.trace_summary(str(d), str(out), 1, 2) == 18
    text = out.read_text()
    assert "| `gemm_fp8_tall_kernel<0>` | side |" in text
    # the call shown is the last of region 1: index 2*1 + 2 - 1 = 3, durations 400 ns
    assert "| 0.4 |" in text
    with pytest.raises(SystemExit):
        bench.trace_summary(str(d), str(out), 2, 2)
