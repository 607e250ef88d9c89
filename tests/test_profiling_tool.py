"""Host-side check of the rocprofv3 summariser (no GPU, no profiler): synthetic
counter and trace files in rocprofv3's CSV layout go in, and the calibrated
counter bytes, the summaries and the hbm_counters.json entries come out. The
calibration scales FETCH_SIZE and WRITE_SIZE so that the runtime's 1 GiB copy
reads as 1 GiB read plus 1 GiB written."""
import csv
import gzip
import json
import os

import bench
from gated_deltanet_speculative_gdn_amd import profiling as PR

VERIFY = "void gdn::(anonymous namespace)::verify_kernel<float, false, 2, 256, 4, false>(gdn::VerifyParams)"
COMMIT = "void gdn::(anonymous namespace)::commit_kernel<float, false, 8, false, false, false>(gdn::CommitParams)"
COPY = "__amd_rocclr_copyBuffer"


def write_counters(path, counter, rows, compress=False):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    opener = (lambda p: gzip.open(p + ".gz", "wt", newline="")) if compress else (lambda p: open(p, "w", newline=""))
    with opener(path) as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for name, value in rows:
            w.writerow({"Kernel_Name": name, "Counter_Name": counter, "Counter_Value": value})


def test_summarize_calibrates_and_replaces_entries(tmp_path, monkeypatch):
    out, prof = tmp_path / "out", tmp_path / "profiles"
    prof.mkdir()
    monkeypatch.setattr(PR, "ROOT", str(tmp_path))
    monkeypatch.setattr(PR, "OUT", "out")
    monkeypatch.setattr(PR, "PROFILES", str(prof))
    monkeypatch.setattr(PR, "COUNTERS_JSON", str(prof / "hbm_counters.json"))
    d = out / "prof_t"
    # the copy of 1 GiB reads as half its bytes in FETCH_SIZE and all of them in WRITE_SIZE
    write_counters(str(d / "fetch" / "fetch_counter_collection.csv"), "FETCH_SIZE",
                   [(COPY, 524288), (COPY, 100), (VERIFY, 1000), (VERIFY, 1000), (COMMIT, 40000)],
                   compress=True)
    write_counters(str(d / "write" / "write_counter_collection.csv"), "WRITE_SIZE",
                   [(COPY, 1048576), (VERIFY, 300), (VERIFY, 300), (COMMIT, 80000)])
    alg = {"verify": 2_300_000, "commit_all_layers": 164_000_000}
    line = {"kernels": {k: {"algorithmic_bytes_per_launch": v, "us_per_launch": 1.0} for k, v in alg.items()},
            "steps": 20, "warmup": 5, "ms_per_step": 1.5}
    (d / "trace.json").write_text("log line\n" + json.dumps(line) + "\n")
    (d / "trace20.json").write_text(json.dumps(line) + "\n")
    (d / "trace20").mkdir()
    with open(d / "trace20" / "trace_kernel_stats.csv", "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Name", "Calls", "AverageNs", "MinNs", "MaxNs"])
        w.writeheader()
        w.writerow({"Name": VERIFY, "Calls": 10, "AverageNs": 28000, "MinNs": 27000, "MaxNs": 29000})
    # an entry of another workload survives, the old entry of this one is replaced
    other = {"kernel": "verify", "workload": "other", "state_dtype": "fp32", "bytes_per_launch": 1}
    stale = {"kernel": "verify", "workload": "wl", "state_dtype": "fp32", "bytes_per_launch": 2}
    (prof / "hbm_counters.json").write_text(json.dumps([other, stale]))

    PR.summarize("t", "wl", "fp32", 3)

    entries = json.loads((prof / "hbm_counters.json").read_text())
    assert other in entries and stale not in entries
    mine = {e["kernel"]: e for e in entries if e["workload"] == "wl"}
    assert abs(mine["verify"]["fetch_factor"] - 2.0) < 1e-12 and mine["verify"]["write_factor"] == 1.0
    # verify: (1000 x 2 + 300 x 1) KiB per dispatch; commit: (40000 x 2 + 80000) KiB
    assert mine["verify"]["bytes_per_launch"] == 2300 * 1024
    assert mine["commit_all_layers"]["bytes_per_launch"] == 160000 * 1024
    assert mine["verify"]["kernel_source_hash"] == bench.source_hash("verify")
    assert mine["verify"]["algorithmic_bytes_per_launch"] == alg["verify"]
    md = (prof / "hbm_counters_wl.md").read_text()
    assert "FETCH_SIZE x 2.000 + WRITE_SIZE x 1.000" in md
    assert "profiling run t wl fp32 3" in md
    assert "| 28.00 |" in (prof / "kernel_trace_wl.md").read_text()


def test_open_prefers_the_newer_of_plain_and_compressed(tmp_path):
    p = tmp_path / "x.csv"
    p.write_text("old")
    os.utime(p, (1, 1))
    with gzip.open(str(p) + ".gz", "wt") as f:
        f.write("new")
    with PR._open(str(p)) as f:
        assert f.read() == "new"
    os.utime(str(p) + ".gz", (0, 0))
    with PR._open(str(p)) as f:
        assert f.read() == "old"
