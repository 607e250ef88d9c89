"""Host-side checks of bench.py that need no GPU: a request for more than one
GPU is refused with a message (the path has no collective; one GPU's share
is the measured unit), an unknown workload name is rejected, and the stored
counter traffic is reported only for the configuration it was taken on."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run_bench(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT,
                          capture_output=True, text=True, timeout=300)


def test_more_than_one_gpu_is_refused():
    r = run_bench("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_unknown_workload_is_rejected():
    r = run_bench("--workload", "no_such_workload")
    assert r.returncode != 0
    assert r.stdout == ""


def test_counter_traffic_only_for_the_configuration_it_was_taken_on(tmp_path):
    """Stored rocprofv3 bytes are reported only for a run of the same kernel,
    kernel source, workload and algorithmic launch bytes; any other run
    reports no traffic rather than another configuration's."""
    import json
    sys.path.insert(0, ROOT)
    import bench
    p = tmp_path / "c.json"
    rec = {"kernel": "commit_all_layers", "workload": "mtp_decode_l48_b64_d4",
           "kernel_source_hash": bench.source_hash("commit_all_layers"),
           "bytes_per_launch": 1001, "algorithmic_bytes_per_launch": 1000}
    ver = dict(rec, kernel="verify", kernel_source_hash=bench.source_hash("verify"),
               bytes_per_launch=21, algorithmic_bytes_per_launch=20)
    p.write_text(json.dumps([rec, ver]))
    tr = bench.counters_traffic
    assert tr("commit_all_layers", "mtp_decode_l48_b64_d4", 1000, path=p) == 1001
    assert tr("verify", "mtp_decode_l48_b64_d4", 20, path=p) == 21
    assert tr("verify", "mtp_decode_l48_b64_d4", 1000, path=p) is None          # another kernel's entry
    assert tr("commit_all_layers", "mtp_decode_l48_b64_d4", 500, path=p) is None  # e.g. bf16 state
    assert tr("commit_all_layers", "all_layer_commit_l36_b16", 1000, path=p) is None
    p.write_text(json.dumps([dict(rec, kernel_source_hash=bench.source_hash("verify"))]))
    assert tr("commit_all_layers", "mtp_decode_l48_b64_d4", 1000, path=p) is None  # other source
    p.write_text(json.dumps(rec))                                                  # not a list
    assert tr("commit_all_layers", "mtp_decode_l48_b64_d4", 1000, path=p) is None
    assert tr("commit_all_layers", "mtp_decode_l48_b64_d4", 1000, path=tmp_path / "none.json") is None
    # every committed entry matches its kernel's current source
    stored = json.load(open(bench.COUNTERS_FILE))
    assert {(e["kernel"], e["workload"]) for e in stored} >= {
        ("commit_all_layers", "mtp_decode_l48_b64_d4"), ("verify", "ring_align_l36_b256_l16")}
    for e in stored:
        assert tr(e["kernel"], e["workload"], e["algorithmic_bytes_per_launch"]) == e["bytes_per_launch"]
