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
    """The stored rocprofv3 commit bytes are reported only for a run of the same
    kernel source, workload and algorithmic launch bytes; any other run reports
    no traffic rather than another configuration's."""
    import json
    sys.path.insert(0, ROOT)
    import bench
    p = tmp_path / "c.json"
    rec = {"workload": "mtp_decode_l48_b64_d4", "kernel_source_hash": bench.source_hash(),
           "bytes_per_launch": 1001, "algorithmic_bytes_per_launch": 1000}
    p.write_text(json.dumps(rec))
    assert bench.counters_traffic("mtp_decode_l48_b64_d4", 1000, path=p) == 1001
    assert bench.counters_traffic("mtp_decode_l48_b64_d4", 500, path=p) is None   # e.g. bf16 state
    assert bench.counters_traffic("all_layer_commit_l36_b16", 1000, path=p) is None
    p.write_text(json.dumps(dict(rec, kernel_source_hash="0" * 16)))
    assert bench.counters_traffic("mtp_decode_l48_b64_d4", 1000, path=p) is None
    assert bench.counters_traffic("mtp_decode_l48_b64_d4", 1000, path=tmp_path / "none.json") is None
    # the committed summary matches the default workload's commit on the current source
    stored = json.load(open(bench.COUNTERS_FILE))
    assert bench.counters_traffic(stored["workload"], stored["algorithmic_bytes_per_launch"]) \
        == stored["bytes_per_launch"]
