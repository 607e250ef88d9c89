"""rocprofv3 driver for the benchmark: kernel traces, calibrated HBM counter
bytes and SQ instruction counters of one workload, and the text summaries
under profiles/ (plus profiles/hbm_counters.json, which bench.py reads to
report the counter bytes of a launch beside its algorithmic bytes).

A measurement tool, not part of the library's call path. Usage, from the
repository root on a machine with the GPU (each rocprofv3 pass is a process of
its own; counter passes never mix with tracing):

    python -m gated_deltanet_speculative_gdn_amd.profiling run TAG WORKLOAD DTYPE STEPS
    python -m gated_deltanet_speculative_gdn_amd.profiling sq TAG WORKLOAD DTYPE
    python -m gated_deltanet_speculative_gdn_amd.profiling summarize TAG WORKLOAD DTYPE STEPS

`run` writes raw rocprofv3 output under gpurun_out/prof_TAG (large per-dispatch
CSVs are compressed there); `summarize` reads it and writes
profiles/kernel_trace_<workload>[_bf16].md, profiles/hbm_counters_<...>.md and
the workload's entries of profiles/hbm_counters.json.

Counter calibration: FETCH_SIZE and WRITE_SIZE are scaled by what they read for
the runtime's 1 GiB device-to-device copy that bench.py --copy-probe-mib 1024
issues in the same run (1 GiB read and 1 GiB written); the library's own copy
and write probe kernels in the same run cross-check the factors.
"""
from __future__ import annotations

import collections
import csv
import gzip
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OUT = "gpurun_out"
PROFILES = os.path.join(ROOT, "profiles")
COUNTERS_JSON = os.path.join(PROFILES, "hbm_counters.json")
SQ_PASSES = (
    ("sq1", "SQ_INSTS_VALU SQ_ACTIVE_INST_VALU SQ_INSTS_LDS SQ_WAVES SQ_INSTS_SALU GRBM_GUI_ACTIVE"),
    ("sq2", "SQ_WAVE_CYCLES SQ_BUSY_CYCLES SQ_WAIT_INST_ANY SQ_INSTS_VMEM SQ_WAIT_ANY"),
)


def bench_args(workload: str, dtype: str, steps: int, warmup: int, probe_mib: int) -> list:
    return ["bench.py", "--workload", workload, "--state-dtype", dtype, "--steps", str(steps),
            "--warmup", str(warmup), "--no-cpu", "--no-native", "--no-all-configs",
            "--copy-probe-mib", str(probe_mib)]


def _rocprof(opts: list, outdir: str, name: str, args: list, log: str) -> None:
    cmd = ["timeout", "-k", "10", "300", "rocprofv3", *opts, "--output-format", "csv", "-d",
           outdir, "-o", name, "--", sys.executable, *args]
    print(" ".join(cmd[4:]), flush=True)
    with open(log + ".json", "w") as fo, open(log + ".err", "w") as fe:
        r = subprocess.run(cmd, cwd=ROOT, stdout=fo, stderr=fe, env=dict(os.environ, TMPDIR="/tmp"))
    if r.returncode != 0:
        raise SystemExit(f"rocprofv3 failed ({r.returncode}); see {log}.err")


def _compress(outdir: str) -> None:
    """Drop the per-dispatch kernel trace (only the stats are summarised) and
    gzip the other large CSVs, so the raw output stays small."""
    for dirpath, _, files in os.walk(outdir):
        for f in files:
            p = os.path.join(dirpath, f)
            if f.endswith("_kernel_trace.csv"):
                os.remove(p)
            elif f.endswith(".csv") and os.path.getsize(p) > 512 << 10:
                with open(p, "rb") as src, gzip.open(p + ".gz", "wb", 9) as dst:
                    dst.write(src.read())
                os.remove(p)


def run(tag: str, workload: str, dtype: str, steps: int) -> None:
    """Kernel trace with stats, FETCH_SIZE and WRITE_SIZE passes (with the
    1 GiB calibration copy), and a 20-step trace for the per-kernel averages."""
    o = os.path.join(OUT, f"prof_{tag}")
    os.makedirs(os.path.join(ROOT, o), exist_ok=True)
    b = bench_args(workload, dtype, steps, 1, 1024)
    _rocprof(["--kernel-trace", "--stats"], f"{o}/trace", "trace", b, f"{ROOT}/{o}/trace")
    _rocprof(["--pmc", "FETCH_SIZE"], f"{o}/fetch", "fetch", b, f"{ROOT}/{o}/fetch")
    _rocprof(["--pmc", "WRITE_SIZE"], f"{o}/write", "write", b, f"{ROOT}/{o}/write")
    t20 = 3 if workload.startswith("ring") else 20     # the ring's step is 16 verify passes
    _rocprof(["--kernel-trace", "--stats"], f"{o}/trace20", "trace",
             bench_args(workload, dtype, t20, 5, 0), f"{ROOT}/{o}/trace20")
    _compress(os.path.join(ROOT, o))


def sq(tag: str, workload: str, dtype: str) -> None:
    """The two SQ counter passes over a 2-step run."""
    o = os.path.join(OUT, f"sq_{tag}")
    os.makedirs(os.path.join(ROOT, o), exist_ok=True)
    b = bench_args(workload, dtype, 2, 1, 0)
    for name, counters in SQ_PASSES:
        _rocprof(["--pmc", *counters.split()], f"{o}/{name}", name, b, f"{ROOT}/{o}/{name}")
    _compress(os.path.join(ROOT, o))


def _open(path: str):
    """The CSV at `path` or its compressed copy, whichever was written last."""
    gz = path + ".gz"
    if os.path.exists(gz) and (not os.path.exists(path) or
                               os.path.getmtime(gz) >= os.path.getmtime(path)):
        return gzip.open(gz, "rt")
    return open(path)


def _counters(path: str) -> dict:
    agg = collections.defaultdict(lambda: collections.defaultdict(list))
    with _open(path) as f:
        for row in csv.DictReader(f):
            agg[row["Kernel_Name"]][row["Counter_Name"]].append(float(row["Counter_Value"]))
    return agg


def _last_json(path: str) -> dict:
    with open(path) as f:
        return json.loads(f.read().strip().splitlines()[-1])


def _short(name: str) -> str:
    for a in ("void gdn::(anonymous namespace)::", "gdn::(anonymous namespace)::",
              "(gdn::VerifyParams)", "(gdn::CommitParams)", "(gdn::PlanParams)"):
        name = name.replace(a, "")
    return name


def summarize(tag: str, workload: str, dtype: str, steps: int) -> list:
    """Write the kernel-trace and HBM-counter summaries of one `run` and
    replace the workload's entries in profiles/hbm_counters.json."""
    sys.path.insert(0, ROOT)
    import bench
    o = os.path.join(ROOT, OUT, f"prof_{tag}")
    mod = "python -m gated_deltanet_speculative_gdn_amd.profiling"
    fe = {kn: c["FETCH_SIZE"] for kn, c in _counters(f"{o}/fetch/fetch_counter_collection.csv").items()}
    wr = {kn: c["WRITE_SIZE"] for kn, c in _counters(f"{o}/write/write_counter_collection.csv").items()}
    cf = [x for x in fe["__amd_rocclr_copyBuffer"] if x > 500000]
    cw = [x for x in wr["__amd_rocclr_copyBuffer"] if x > 1000000]
    ff = 1048576 / (sum(cf) / len(cf))
    wf = 1048576 / (sum(cw) / len(cw))
    k = _last_json(f"{o}/trace.json")["kernels"]
    d20 = _last_json(f"{o}/trace20.json")
    k20 = d20["kernels"]
    b = " ".join(bench_args(workload, dtype, steps, 1, 1024))
    cmds = [f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d gpurun_out/prof_{tag}/fetch -o fetch -- python3 {b}",
            f"rocprofv3 --pmc WRITE_SIZE --output-format csv -d gpurun_out/prof_{tag}/write -o write -- python3 {b}"]
    entries, rows = [], []
    for name, sub in (("verify", "verify_kernel<"), ("commit_all_layers", "commit_kernel<")):
        ks = [n for n in fe if sub in n and "true, 2, 256" not in n]
        assert len(ks) == 1, ks
        kn = ks[0]
        f = sum(fe[kn]) / len(fe[kn])
        w = sum(wr[kn]) / len(wr[kn])
        by = (f * ff + w * wf) * 1024
        alg = k[name]["algorithmic_bytes_per_launch"]
        entries.append(dict(kernel=name, workload=workload, state_dtype=dtype,
                            kernel_source_hash=bench.source_hash(name),
                            bytes_per_launch=int(round(by)), algorithmic_bytes_per_launch=alg,
                            fetch_kib=f, write_kib=w, fetch_factor=ff, write_factor=wf,
                            commands=cmds))
        rows.append(f"| {_short(kn)} | {len(fe[kn])} | {f:.0f} | {w:.0f} | {by / 1e9:.4f} GB | "
                    f"{alg / 1e9:.4f} GB | {by / alg:.4f} |")
    for pk, label, alg in (("probe_kernel<1>", "probe_kernel<1> (write probe, 1 GiB)", 1 << 30),
                           ("probe_kernel<2>", "probe_kernel<2> (copy probe, 1 GiB)", 2 << 30)):
        ks = [n for n in fe if pk in n]
        if len(ks) == 1:
            kn = ks[0]
            f = sum(fe[kn]) / len(fe[kn])
            w = sum(wr[kn]) / len(wr[kn])
            by = (f * ff + w * wf) * 1024
            rows.append(f"| {label} | {len(fe[kn])} | {f:.0f} | {w:.0f} | {by / 1e9:.4f} GB | "
                        f"{alg / 1e9:.4f} GB | {by / alg:.4f} |")
    title = "fp32 state" if dtype == "fp32" else "bf16 state"
    counters_md = [
        f"# rocprofv3 HBM counters: {workload} ({title})", "",
        "Made by (repo root, one MI355X; one counter per rocprofv3 run):", "",
        f"    {mod} run {tag} {workload} {dtype} {steps}",
        f"    {mod} summarize {tag} {workload} {dtype} {steps}", "",
        "whose counter passes are:", ""] + ["    " + c for c in cmds] + ["",
        "Calibration: bench.py --copy-probe-mib 1024 copies 1 GiB = 1048576 KiB (read and written) with the "
        "runtime's copy kernel;",
        f"in these runs the counters read FETCH_SIZE {1048576 / ff:.0f} KiB and WRITE_SIZE {1048576 / wf:.0f} KiB "
        f"per copy, so bytes = FETCH_SIZE x {ff:.3f} + WRITE_SIZE x {wf:.3f} (KiB).", "",
        "| kernel | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | HBM bytes (calibrated) | algorithmic bytes | ratio |",
        "|---|---|---|---|---|---|---|"] + rows + ["",
        "Per-dispatch averages. The probe rows (the library's own streaming kernels, bytes known) cross-check "
        "the calibration. Kernel source hashes: " +
        ", ".join(f"{e['kernel']} {e['kernel_source_hash']}" for e in entries) + ".", ""]
    with _open(f"{o}/trace20/trace_kernel_stats.csv") as fh:
        stats = [r for r in csv.DictReader(fh) if "gdn::" in r["Name"]]
    bt = " ".join(bench_args(workload, dtype, d20["steps"], d20["warmup"], 0))
    trace_md = [
        f"# rocprofv3 kernel trace: {workload} ({title})", "",
        f"Made by `{mod} run {tag} {workload} {dtype} {steps}` (repo root, one MI355X); its trace pass is:", "",
        f"    rocprofv3 --kernel-trace --stats --output-format csv -d gpurun_out/prof_{tag}/trace20 -o trace -- "
        f"python3 {bt}", "",
        "| kernel | calls | avg us | min us | max us |", "|---|---|---|---|---|"]
    for r in stats:
        trace_md.append(f"| {_short(r['Name'])} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                        f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} |")
    trace_md += ["", f"Same kernels timed by HIP events inside bench.py over the {d20['steps']} timed steps of "
                 f"the same profiled run: verify {k20['verify']['us_per_launch']:.2f} us/launch, commit "
                 f"{k20['commit_all_layers']['us_per_launch']:.1f} us/launch; step {d20['ms_per_step']:.3f} ms. "
                 "The profiler's averages also count the warm-up launches.", ""]
    fname = workload if dtype == "fp32" else f"{workload}_{dtype}"
    with open(os.path.join(PROFILES, f"kernel_trace_{fname}.md"), "w") as fh:
        fh.write("\n".join(trace_md))
    with open(os.path.join(PROFILES, f"hbm_counters_{fname}.md"), "w") as fh:
        fh.write("\n".join(counters_md))
    try:
        with open(COUNTERS_JSON) as fh:
            cur = json.load(fh)
    except (OSError, ValueError):
        cur = []
    cur = [e for e in cur if not (e["workload"] == workload and e.get("state_dtype", "fp32") == dtype)]
    with open(COUNTERS_JSON, "w") as fh:
        json.dump(cur + entries, fh, indent=1)
    return rows


def main(argv: list) -> None:
    if len(argv) < 4 or argv[0] not in ("run", "sq", "summarize"):
        raise SystemExit(__doc__)
    cmd, tag, workload, dtype = argv[:4]
    if cmd == "run":
        run(tag, workload, dtype, int(argv[4]))
    elif cmd == "sq":
        sq(tag, workload, dtype)
    else:
        for r in summarize(tag, workload, dtype, int(argv[4])):
            print(r)


if __name__ == "__main__":
    main(sys.argv[1:])
