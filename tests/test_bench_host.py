"""Host logic of bench.py: the counter summary's calibration by the 1 GiB copy,
and the lookup of committed HBM traffic per workload and kernel sources."""
import csv
import json

import pytest

import bench

pytestmark = pytest.mark.filterwarnings("ignore")

FIELDS = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]


def write_counters(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for i, (k, c, v) in enumerate(rows):
            w.writerow({"Dispatch_Id": i, "Kernel_Name": k, "Counter_Name": c, "Counter_Value": v})


def test_summarize_scales_by_the_calibration_copy(tmp_path, capsys):
    # the copy moves 1 GiB = 2^20 KiB; its counter reads half of that, so every
    # FETCH_SIZE is scaled x2; two dispatches of the kernel average to 3 GiB counted
    d = tmp_path / "run"
    d.mkdir()
    gib = 1 << 20
    write_counters(d / "x_counter_collection.csv", [
        ("__amd_rocclr_copyBuffer(void*)", "FETCH_SIZE", gib / 2),
        ("__amd_rocclr_copyBuffer(void*)", "FETCH_SIZE", 4.0),   # a small copy: not the calibration
        ("void dion::k_gemm16<256, 1, 1, 0, true>(dion::MatDesc const*)", "FETCH_SIZE", 2 * gib),
        ("void dion::k_gemm16<256, 1, 1, 0, true>(dion::MatDesc const*)", "FETCH_SIZE", 4 * gib),
    ])
    bench.summarize(str(d))
    out = capsys.readouterr().out
    lines = [json.loads(l[8:]) for l in out.splitlines() if l.startswith("TRAFFIC {")]
    assert len(lines) == 1
    t = lines[0]
    assert t["kernel"] == "dion::k_gemm16<256, 1, 1, 0, true>" and t["counter"] == "FETCH_SIZE"
    assert t["scale"] == pytest.approx(2.0)
    assert t["bytes_per_dispatch"] == pytest.approx(6.0 * (1 << 30))
    assert t["sources_sha256"] == bench.sources_sha256()


def test_traffic_lookup_by_workload_and_sources(tmp_path, monkeypatch):
    sha = bench.sources_sha256()
    k = "dion::k_gemm16<256, 1, 1, 0, true>"
    f = tmp_path / "t.txt"
    f.write_text("header\n" + "\n".join("TRAFFIC " + json.dumps(x) for x in [
        {"kernel": k, "counter": "FETCH_SIZE", "bytes_per_dispatch": 5.0, "scale": 2.0, "sources_sha256": sha},
        {"kernel": k, "counter": "WRITE_SIZE", "bytes_per_dispatch": 2.0, "scale": 1.0, "sources_sha256": sha},
        {"kernel": "dion::other", "counter": "FETCH_SIZE", "bytes_per_dispatch": 9.0, "scale": 2.0,
         "sources_sha256": "0" * 64},
        {"kernel": "dion::other", "counter": "WRITE_SIZE", "bytes_per_dispatch": 9.0, "scale": 1.0,
         "sources_sha256": "0" * 64},
    ]) + "\n")
    monkeypatch.setattr(bench, "TRAFFIC_FILES", {"llama3_8b": str(f)})
    assert bench.traffic_for(k, "llama3_8b") == 7.0
    assert bench.traffic_for("dion::other", "llama3_8b") is None      # taken on other kernel sources
    assert bench.traffic_for(k, "llama3_70b") is None                 # no counters for that workload
    assert bench.traffic_for("dion::missing", "llama3_8b") is None


def test_gpus_above_one_is_refused(monkeypatch, capsys):
    monkeypatch.setattr("sys.argv", ["bench.py", "--gpus", "2"])
    with pytest.raises(SystemExit) as e:
        bench.main()
    assert e.value.code == 2
    assert "one GPU only" in capsys.readouterr().out


def test_summarize_kernel_stats_with_warm_average(tmp_path, capsys):
    d = tmp_path / "trace"
    d.mkdir()
    with open(d / "x_kernel_stats.csv", "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage"])
        w.writeheader()
        w.writerow({"Name": "void dion::k_select(int)", "Calls": 3, "TotalDurationNs": 6000, "AverageNs": 2000,
                    "Percentage": 100.0})
    with open(d / "x_kernel_trace.csv", "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        for start, end in ((500, 1500), (0, 3000), (4000, 5000)):   # out of order: the first launch is the slow one
            w.writerow({"Kernel_Name": "void dion::k_select(int)", "Start_Timestamp": start, "End_Timestamp": end})
    bench.summarize(str(d))
    line = [l for l in capsys.readouterr().out.splitlines() if l.startswith("dion::k_select")][0]
    assert line.split()[-1] == "1.0"   # (1000 + 1000) / 2 ns after the first launch, in us
    assert line.split()[3] == "2.0"
