"""Benchmark of the verify + commit hot path on one MI355X.

One step = one MTP decode step of the workload: gdn_verify for every layer
(captured once in a HIP graph and replayed, as the layer launches run inside a
captured decode graph) followed by one gdn_commit_all_layers launch (outside
the graph, as the commit runs after sampling). Inputs are seeded synthetic
tensors already resident in HBM. The commit works in place, so each step
starts from the previous step's committed state; its cost does not depend on
the values.

Prints one JSON line: state-updates/s (one update = one token applied to one
128x128 head; verify counts every window token, commit every accepted token),
per-kernel times from HIP events on the launch stream, the roofline of the
step's dominant kernel (the one with the larger share of the step) against the
8 TB/s HBM peak, with its rocprofv3 counter bytes when they were taken on this
configuration and kernel source, the native snapshot-every-token baseline
timed the same way, the CPU oracle timed on the host's cores, and under
"all_configs" the same step timing for every workload (fp32 state, and the
batch-64 workload on a bf16 pool as well), each with the library's read probe
timed over the bytes of one of its verify launches. Per-launch times are the means of
the per-step HIP-event times (what rocprofv3's kernel averages match), with
their medians beside them.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import gated_deltanet_speculative_gdn_amd as G  # noqa: E402
from gated_deltanet_speculative_gdn_amd import workloads as W  # noqa: E402

HBM_PEAK_GBS = 8000.0
REC_TOKEN_BYTES = (128 + 128 + 1) * 4           # correction, key, gate (fp32)
PAYLOAD_TOKEN_BYTES = (128 + 128) * 2 + 2 * 4    # raw key, raw value (bf16), gate, beta (fp32)
CHANNEL_TOKEN_BYTES = (128 + 128 + 128) * 4      # correction, key, per-channel decays (fp32)
CHANNEL_GATE_BYTES = 128 * 4 + 4                 # per-channel log-decays and beta, per head
COUNTERS_FILE = os.path.join(ROOT, "profiles", "hbm_counters.json")
_CSRC = "gated_deltanet_speculative_gdn_amd/csrc/"
KERNEL_SOURCES = {
    "commit_all_layers": [_CSRC + "gdn_commit.hip", _CSRC + "gdn_device.hpp", _CSRC + "gdn_kernels.hpp",
                          _CSRC + "gdn_divide.hpp"],
    "verify": [_CSRC + "gdn_verify.hip", _CSRC + "gdn_device.hpp", _CSRC + "gdn_kernels.hpp",
               _CSRC + "gdn_divide.hpp"],
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_hash(kernel: str = "commit_all_layers") -> str:
    """Hash of one kernel's sources with comments and blank space removed, so
    that the stored counters stay valid across comment edits."""
    import re
    h = hashlib.sha256()
    for p in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, p)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def i32(x):
    return torch.as_tensor(np.ascontiguousarray(x, dtype=np.int32), device="cuda")


class Step:
    """Device buffers and launch closures for one workload."""

    def __init__(self, wl, raw_gates=False, out_dtype=torch.float32, conv=None,
                 record_kind=G.RECORD_CORRECTION):
        # per-key-channel decays go with their own record kind
        self.a_ch = W.make_channel_decays(wl, device="cuda") \
            if record_kind == G.RECORD_CHANNEL else None
        s = wl.spec
        self.wl, self.s = wl, s
        self.rec = G.Pools.alloc_records(s.layers, s.rows, s.hv, s.rec_tokens,
                                         record_kind=record_kind)
        self.pools = G.Pools(wl.state, self.rec, s.hk, s.rec_tokens, record_kind)
        self.out = torch.zeros((s.layers, wl.tokens, s.hv, s.dv), dtype=out_dtype, device="cuda")
        self.rg = W.make_raw_gates(wl, device="cuda") if raw_gates else None
        self.conv = G.ConvPools(conv.state, conv.x) if conv is not None else None
        self.err = torch.zeros(1, dtype=torch.int32, device="cuda")
        self.slot = i32(wl.state_slot)
        self.rec_slot = i32(wl.rec_slot)
        self.tok = i32(wl.tok_start)
        self.win = i32(wl.win_len)
        self.n = i32(wl.n_accept)
        self.snaps = None
        self.plan = None
        if s.ring_steps:
            # align-mode slots of the ring's flush, planned once on the device
            self.plan = [torch.empty(s.rows, dtype=torch.int32, device="cuda") for _ in range(4)]
            G.gdn_align_plan(i32(wl.p0), self.n, i32(wl.block_table), s.block, s.rec_tokens,
                             *self.plan, err_flags=self.err)
            self.ring_base = [i32(np.full(s.rows, j)) for j in range(s.ring_steps)]

    def gates(self, layer):
        """(a, b, keyword arguments) of the layer's verify: log-gate and beta,
        or the raw projections with the per-head gate parameters."""
        if self.a_ch is not None:
            return self.a_ch[layer], self.wl.beta[layer], {}
        if self.rg is None:
            return self.wl.a[layer], self.wl.beta[layer], {}
        rg = self.rg
        return rg.a[layer], rg.b[layer], {"A_log": rg.A_log[layer], "dt_bias": rg.dt_bias[layer]}

    def verify_all(self):
        wl, s = self.wl, self.s
        if s.ring_steps:
            # one single-token verify per layer and ring step, pending records first
            for j in range(s.ring_steps):
                sl = slice(j * s.rows, (j + 1) * s.rows)
                for layer in range(s.layers):
                    a, b, kw = self.gates(layer)
                    G.gdn_verify(self.pools, layer, self.slot, self.rec_slot, self.tok, self.win,
                                 self.ring_base[j], wl.q(layer)[sl], wl.k(layer)[sl],
                                 wl.v(layer)[sl], a[sl], b[sl], self.out[layer, sl],
                                 err_flags=self.err, **kw)
            return
        for layer in range(s.layers):
            a, b, kw = self.gates(layer)
            G.gdn_verify(self.pools, layer, self.slot, self.rec_slot, self.tok, self.win, None,
                         wl.q(layer), wl.k(layer), wl.v(layer), a, b, self.out[layer],
                         err_flags=self.err, **kw)

    def commit(self):
        if self.plan is not None:
            src, dst, bl, bs = self.plan
            G.gdn_commit_all_layers(self.pools, src, dst, self.rec_slot, self.n, bl, bs,
                                    err_flags=self.err)
            return
        if self.conv is None:
            G.gdn_commit_all_layers(self.pools, self.slot, self.slot, self.rec_slot, self.n,
                                    err_flags=self.err)
        else:
            G.gdn_commit_all_layers_conv(self.pools, self.conv, self.slot, self.slot,
                                         self.rec_slot, self.n, conv_tok_start=self.tok,
                                         err_flags=self.err)

    def native_all(self):
        wl, s = self.wl, self.s
        if self.snaps is None:
            self.snaps = [torch.empty((s.rows, s.hv, s.rec_tokens, 128, 128),
                                      dtype=wl.state_dtype, device="cuda")
                          for _ in range(s.layers)]
        for layer in range(s.layers):
            a, b, kw = self.gates(layer)
            G.gdn_native_window(self.pools, layer, self.slot, self.tok, self.win, wl.q(layer),
                                wl.k(layer), wl.v(layer), a, b, self.out[layer],
                                self.snaps[layer], err_flags=self.err, **kw)

    def native_accept(self):
        G.gdn_native_accept(self.pools, self.snaps, self.slot, self.n, err_flags=self.err)


def accounting(wl, out_bytes=4, raw_gates=False, conv=None, rec_bytes=REC_TOKEN_BYTES,
               gate_bytes=8):
    """Update counts and algorithmic HBM bytes of one step (out_bytes: bytes
    per output element; raw gates add the per-head parameters; conv: the
    short-conv states compacted in the commit launch)."""
    s = wl.spec
    sb = 128 * 128 * (4 if wl.state_dtype == torch.float32 else 2)
    real = (wl.state_slot >= 0) & (wl.win_len > 0)
    w = wl.win_len[real].astype(np.int64)
    n = wl.n_accept[real].astype(np.int64)
    steps = max(s.ring_steps, 1)
    verify_updates = int(s.layers * s.hv * w.sum() * steps)
    commit_updates = int(s.layers * s.hv * n.sum())
    per_tok = s.hk * 2 * 128 * 2 + s.hv * (128 * 2 + gate_bytes + 128 * out_bytes + rec_bytes)
    verify_bytes_layer = int(real.sum() * s.hv * sb + w.sum() * per_tok + (s.hv * 8 if raw_gates else 0))
    if s.ring_steps:
        # average launch of the ring: step j also reads j pending records per head
        pending = sum(range(s.ring_steps)) / s.ring_steps
        verify_bytes_layer += int(real.sum() * s.hv * pending * rec_bytes)
    commit_bytes = int(s.layers * s.hv * ((n > 0).sum() * 2 * sb + n.sum() * rec_bytes))
    if s.ring_steps:
        # align flush: a boundary state is written for windows that cross a block
        t_b = np.where(wl.p0 % s.block == 0, s.block, s.block - wl.p0 % s.block)
        commit_bytes += int(s.layers * s.hv * (t_b < wl.n_accept).sum() * sb)
    if conv is not None:
        Ls, C = conv.state.shape[2], conv.state.shape[3]
        row = C * conv.state.element_size()
        # per live row and layer: read L_s state rows and n inputs, write L_s rows
        commit_bytes += int(s.layers * ((n > 0).sum() * 2 * Ls * row + n.sum() * row))
    native_bytes_layer = int(real.sum() * s.hv * sb + w.sum() * (per_tok - s.hv * rec_bytes)
                             + w.sum() * s.hv * sb)
    accept_bytes = int(s.layers * s.hv * (n > 0).sum() * 2 * sb)
    return dict(verify_updates=verify_updates, commit_updates=commit_updates,
                verify_bytes_per_launch=verify_bytes_layer, commit_bytes_per_launch=commit_bytes,
                native_bytes_per_launch=native_bytes_layer, accept_bytes_per_launch=accept_bytes)


def timed_loop(steps, graph_fn, eager_fn, graph_launches):
    """Run `steps` steps of graph replay + one eager launch. Returns wall ms
    per step (host clock over all steps, bracketed by synchronisation) and,
    from HIP events on the launch stream, per-step arrays (ms) of the graph
    part and of the eager launch."""
    sync = torch.cuda.synchronize
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
           torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    sync()
    t0 = time.perf_counter()
    for e0, e1, e2 in ev:
        e0.record()
        graph_fn()
        e1.record()
        eager_fn()
        e2.record()
    sync()
    wall = (time.perf_counter() - t0) * 1e3 / steps
    g_ms = np.array([e0.elapsed_time(e1) for e0, e1, _ in ev])
    c_ms = np.array([e1.elapsed_time(e2) for _, e1, e2 in ev])
    return wall, g_ms, c_ms


def summary_ms(x):
    """Mean and median of per-step event times (ms)."""
    return float(np.mean(x)), float(np.median(x))


def capture(fn):
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    return g


def cpu_baseline(wl, acc, target_s=15.0, a_ch=None):
    """The oracle (plain C, OpenMP over heads) on the same workload: every
    layer's real rows, windows and accepted counts, the whole step repeated
    until about `target_s` seconds of oracle time (the count is fixed from the
    first layer's time). a_ch: per-key-channel log-decays, when the step runs
    with them."""
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    import oracle
    import oracle_pool as OP
    s = wl.spec
    real = np.nonzero((wl.state_slot >= 0) & (wl.win_len > 0))[0]
    nthreads = oracle.default_threads()
    keep = np.repeat(wl.n_accept[real], s.hv)[:, None]

    native = oracle.native_heads if a_ch is None else oracle.native_heads_ch

    def gather(layer):
        g = OP.gather(wl, layer, real)
        if a_ch is not None:
            g["a"] = OP.gather_channel_decays(wl, a_ch, layer, real)
        return g

    def run(g, threads=nthreads):
        t0 = time.perf_counter()
        native(g["S0"], g["w"], g["q"], g["k"], g["v"], g["a"], g["beta"], keep=keep,
               nthreads=threads)
        return time.perf_counter() - t0

    g = gather(0)
    first = run(g)
    reps = max(1, int(np.ceil(target_s / (first * s.layers))))
    spent = first + sum(run(g) for _ in range(reps - 1))
    for layer in range(1, s.layers):
        g = gather(layer)
        spent += sum(run(g) for _ in range(reps))
    updates = reps * (acc["verify_updates"] + acc["commit_updates"])
    # one thread, on the first layer only (a bounded sample of the same rule)
    one = run(gather(0), threads=1)
    single = (acc["verify_updates"] + acc["commit_updates"]) / s.layers / one
    return {"value": updates / spent, "unit": "state-updates/s", "cores": nthreads,
            "kind": "oracle", "seconds": round(spent, 3), "cpu_model": cpu_model(),
            "single_thread_value": single,
            "sample": f"{reps} passes over one full step of {s.name}: {s.layers} layers x "
                      f"{len(real)} rows x {s.hv} heads, native per-token rule with the accepted "
                      f"state kept"}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def counters_traffic(kernel, workload, launch_bytes, path=COUNTERS_FILE):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter
    summaries (a list of entries), or None when no entry was taken on this
    kernel's current source, this workload and this configuration (told apart
    by the launch's algorithmic bytes, which differ with the state dtype, the
    record kind, the conv states and the accepted counts)."""
    try:
        with open(path) as f:
            entries = json.load(f)
    except (OSError, ValueError):
        return None
    if not isinstance(entries, list):
        return None
    for c in entries:
        if (isinstance(c, dict) and c.get("kernel") == kernel and c.get("workload") == workload
                and c.get("kernel_source_hash") == source_hash(kernel)
                and c.get("algorithmic_bytes_per_launch") == int(launch_bytes)
                and c.get("bytes_per_launch")):
            return int(c["bytes_per_launch"])
    return None


def measure(spec, dtype, steps, warmup, gating="log", out_dtype="fp32", record="correction",
            conv=False, accepted="uniform", eager=False):
    """Build one workload on the device, warm up, capture the verify launches
    of a step in a HIP graph and time `steps` steps (graph replay + the eager
    all-layer commit). Returns the workload, its accounting, the Step and the
    timings (means of the per-step event times, which rocprofv3's averages
    match, and medians)."""
    wl = W.make_workload(spec, device="cuda", state_dtype=dtype)
    if accepted == "rates":
        W.draw_acceptance_rate_counts(wl)
    cv = W.make_conv(wl, state_len=3, dtype=torch.bfloat16, device="cuda") if conv else None
    payload = record == "payload"
    channel = gating == "channel"
    acc = accounting(wl, out_bytes=2 if out_dtype == "bf16" else 4, raw_gates=gating == "raw",
                     conv=cv,
                     rec_bytes=(PAYLOAD_TOKEN_BYTES if payload else
                                CHANNEL_TOKEN_BYTES if channel else REC_TOKEN_BYTES),
                     gate_bytes=CHANNEL_GATE_BYTES if channel else 8)
    st = Step(wl, raw_gates=gating == "raw",
              out_dtype=torch.bfloat16 if out_dtype == "bf16" else torch.float32, conv=cv,
              record_kind=(G.RECORD_PAYLOAD if payload else
                           G.RECORD_CHANNEL if channel else G.RECORD_CORRECTION))
    launches = spec.layers * max(spec.ring_steps, 1)
    # warm-up (also loads the code object before capture)
    for _ in range(max(warmup, 1)):
        st.verify_all()
        st.commit()
    torch.cuda.synchronize()
    graph = capture(st.verify_all)
    for _ in range(warmup):
        graph.replay()
        st.commit()
    torch.cuda.synchronize()
    wall, g_ms, c_ms = timed_loop(steps, graph.replay, st.commit, launches)
    assert st.err.item() == 0, f"device row errors {st.err.item()}"
    g_mean, g_med = summary_ms(g_ms)
    c_mean, c_med = summary_ms(c_ms)
    ver_ms, com_ms = g_mean / launches, c_mean
    log(f"{spec.name} {'fp32' if dtype == torch.float32 else 'bf16'}: step {wall:.3f} ms: "
        f"verify graph {g_mean:.3f} ms ({ver_ms * 1e3:.1f} us/layer), commit {com_ms * 1e3:.1f} us")
    updates = acc["verify_updates"] + acc["commit_updates"]
    com_gbs = acc["commit_bytes_per_launch"] / (com_ms / 1e3) / 1e9
    ver_gbs = acc["verify_bytes_per_launch"] / (ver_ms / 1e3) / 1e9
    kernels = {
        "verify": {"us_per_launch": ver_ms * 1e3, "us_per_launch_median": g_med / launches * 1e3,
                   "launches_per_step": launches,
                   "algorithmic_bytes_per_launch": acc["verify_bytes_per_launch"],
                   "GB/s": ver_gbs, "frac_of_peak": ver_gbs / HBM_PEAK_GBS},
        "commit_all_layers": {"us_per_launch": com_ms * 1e3, "us_per_launch_median": c_med * 1e3,
                              "launches_per_step": 1,
                              "algorithmic_bytes_per_launch": acc["commit_bytes_per_launch"],
                              "GB/s": com_gbs, "frac_of_peak": com_gbs / HBM_PEAK_GBS},
    }
    if eager:
        # the same verify launches issued one by one, without the graph (outside
        # the timed step): the host's launch cost per layer shows against the graph's
        eager_steps = max(1, min(steps, 10))
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        ev0.record()
        for _ in range(eager_steps):
            st.verify_all()
        ev1.record()
        torch.cuda.synchronize()
        kernels["verify"]["eager_us_per_launch"] = ev0.elapsed_time(ev1) * 1e3 / (eager_steps * launches)
        assert st.err.item() == 0, f"device row errors {st.err.item()}"
    # the dominant kernel of the step: the one with the larger share of its time
    if c_mean >= g_mean:
        roofline = {"bound": "hbm", "kernel": "commit_all_layers", "achieved": com_gbs,
                    "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": com_gbs / HBM_PEAK_GBS}
    else:
        roofline = {"bound": "hbm", "kernel": "verify", "achieved": ver_gbs,
                    "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": ver_gbs / HBM_PEAK_GBS}
    step_bytes = launches * acc["verify_bytes_per_launch"] + acc["commit_bytes_per_launch"]
    del graph
    return {"wl": wl, "acc": acc, "step": st, "launches": launches, "wall_ms": wall,
            "step_ms_median": float(np.median(g_ms + c_ms)), "updates": updates,
            "kernels": kernels, "roofline": roofline, "step_GB/s": step_bytes / (wall / 1e3) / 1e9}


_PROBE_BUF = {}


def read_probe_at(nbytes, reps=10):
    """Mean time of the library's read probe over `nbytes` (rounded down to the
    probe's chunk), the reads rotating through a 1 GiB buffer so that no
    repetition is served from the 256 MB cache: the read ceiling at the size of
    one verify launch. Returns (bytes, us) or None."""
    size = 1 << 30
    vn = nbytes - nbytes % G.GDN_PROBE_CHUNK
    if not 0 < vn <= size:
        return None
    if "a" not in _PROBE_BUF:
        _PROBE_BUF["a"] = torch.zeros(size // 4, device="cuda")
        _PROBE_BUF["sink"] = torch.empty(size // G.GDN_PROBE_CHUNK * 4, device="cuda")
    a, sink = _PROBE_BUF["a"], _PROBE_BUF["sink"]
    offs = [(i * vn) % (size - vn + 1) // 16 * 16 for i in range(reps)]
    views = [a.view(torch.uint8)[o:o + vn] for o in offs]
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    G.gdn_bandwidth_probe(G.PROBE_READ, views[0], sink, vn)
    torch.cuda.synchronize()
    e0.record()
    for v_ in views:
        G.gdn_bandwidth_probe(G.PROBE_READ, v_, sink, vn)
    e1.record()
    torch.cuda.synchronize()
    return vn, e0.elapsed_time(e1) * 1e3 / reps


def all_configs(steps, warmup):
    """Every workload (fp32 state, and the batch-64 workload on a bf16 pool too)
    timed in this run the same way as the headline, without the native and CPU
    legs: step time, per-launch verify and commit times (means and medians),
    algorithmic GB/s and fraction of the HBM peak, the dominant kernel."""
    out = {}
    for spec in W.ORDERED:
        for dtype in ((torch.float32, torch.bfloat16) if spec is W.MTP_B64 else (torch.float32,)):
            name = spec.name + ("" if dtype == torch.float32 else "_bf16")
            m = measure(spec, dtype, steps, warmup)
            k = m["kernels"]
            out[name] = {
                "ms_per_step": m["wall_ms"], "ms_per_step_median": m["step_ms_median"],
                "state_updates_per_s": m["updates"] / (m["wall_ms"] / 1e3),
                "verify_us_per_launch": k["verify"]["us_per_launch"],
                "verify_us_per_launch_median": k["verify"]["us_per_launch_median"],
                "verify_launches_per_step": m["launches"],
                "verify_GB/s": k["verify"]["GB/s"], "verify_frac": k["verify"]["frac_of_peak"],
                "commit_us": k["commit_all_layers"]["us_per_launch"],
                "commit_us_median": k["commit_all_layers"]["us_per_launch_median"],
                "commit_GB/s": k["commit_all_layers"]["GB/s"],
                "commit_frac": k["commit_all_layers"]["frac_of_peak"],
                "dominant": m["roofline"]["kernel"], "dominant_frac": m["roofline"]["frac"],
            }
            rp = read_probe_at(m["acc"]["verify_bytes_per_launch"])
            if rp is not None:
                out[name]["read_probe_at_verify_bytes_us"] = rp[1]
                out[name]["verify_frac_of_read_probe"] = rp[1] / k["verify"]["us_per_launch"]
            del m
            torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=W.MTP_B64.name, choices=sorted(W.WORKLOADS))
    ap.add_argument("--state-dtype", default="fp32", choices=["fp32", "bf16"])
    ap.add_argument("--gating", default="log", choices=["log", "raw", "channel"],
                    help="log: log-gate and beta given; raw: gates formed in the kernel from "
                         "raw a, b with per-head A_log, dt_bias; channel: one log-decay per key "
                         "channel (records keep the decays per channel)")
    ap.add_argument("--out-dtype", default="fp32", choices=["fp32", "bf16"])
    ap.add_argument("--record", default="correction", choices=["correction", "payload"],
                    help="correction: (delta, k_hat, gate) records, elementwise commit; payload: "
                         "(k, v, gate, beta) records, the commit recomputes the corrections")
    ap.add_argument("--conv", action="store_true",
                    help="also compact bf16 short-conv states (width-4 conv over the mixed "
                         "q/k/v channels) in the commit launch")
    ap.add_argument("--accepted", default="uniform", choices=["uniform", "rates"],
                    help="uniform: accepted counts as the workload draws them; rates: drawn "
                         "from per-position draft acceptance rates (.856/.694/.558 for the "
                         "three drafts of a 4-token window)")
    ap.add_argument("--no-native", action="store_true")
    ap.add_argument("--no-all-configs", action="store_true",
                    help="skip the per-configuration figures of every workload (profiling runs)")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--copy-probe-mib", type=int, default=1024,
                    help="also time a plain device-to-device copy of this size: the measured "
                         "copy ceiling reported beside the kernels, and the counter calibration "
                         "(0 = skip)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (the path "
              "needs no collective and shards by heads, rows or layers)", file=sys.stderr)
        sys.exit(2)
    spec = W.WORKLOADS[args.workload]
    if spec.ring_steps and (args.record == "payload" or args.conv):
        print("the ring workload needs correction records and no conv states", file=sys.stderr)
        sys.exit(2)
    if spec.ring_steps and args.accepted == "rates":
        print("the ring workload's flush commits every ring record", file=sys.stderr)
        sys.exit(2)
    if args.gating == "channel" and args.record == "payload":
        print("per-channel decays keep their own record kind, not the payload record",
              file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)
    G.load_library()
    dtype = torch.float32 if args.state_dtype == "fp32" else torch.bfloat16
    log(f"workload {spec.name} ({spec.description}), state {args.state_dtype}")
    payload = args.record == "payload"
    channel = args.gating == "channel"
    m = measure(spec, dtype, args.steps, args.warmup, gating=args.gating,
                out_dtype=args.out_dtype, record=args.record, conv=args.conv,
                accepted=args.accepted, eager=True)
    wl, acc, st, L, launches = m["wl"], m["acc"], m["step"], spec.layers, m["launches"]
    wall, updates = m["wall_ms"], m["updates"]
    value = updates / (wall / 1e3)
    com_traffic = counters_traffic("commit_all_layers", spec.name, acc["commit_bytes_per_launch"])
    ver_traffic = counters_traffic("verify", spec.name, acc["verify_bytes_per_launch"])
    roofline = dict(m["roofline"])
    roofline["traffic"] = com_traffic if roofline["kernel"] == "commit_all_layers" else ver_traffic
    kern = m["kernels"]
    kern["verify"]["counter_bytes_per_launch"] = ver_traffic
    kern["commit_all_layers"]["counter_bytes_per_launch"] = com_traffic

    result = {
        "metric": "commit+verify state-updates/s and achieved HBM GB/s (% peak), B=64 D=4 48 layers",
        "value": value,
        "unit": "state-updates/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": spec.name, "layers": L, "batch": spec.rows,
                   "padding_rows": spec.pad_rows, "value_heads": spec.hv, "key_heads": spec.hk,
                   "head_dim": 128, "verify_tokens": spec.window, "state_dtype": args.state_dtype,
                   "gating": args.gating, "out_dtype": args.out_dtype, "conv_states": args.conv,
                   "record": "channel" if channel else args.record, "ring_steps": spec.ring_steps, "block": spec.block,
                   "accepted": (f"U{{{spec.n_lo}..{spec.n_hi}}}" if args.accepted == "uniform" else
                                "rates " + "/".join(f"{r:g}" for r in
                                                    W.MTP_ACCEPTANCE_RATES[: spec.window - 1]))},
        "roofline": roofline,
        "kernels": kern,
        "ms_per_step_median": m["step_ms_median"],
        "step_GB/s": m["step_GB/s"],
        "updates_per_step": {"verify": acc["verify_updates"], "commit": acc["commit_updates"]},
        "kernel_source_hash": {k: source_hash(k) for k in KERNEL_SOURCES},
    }
    del m

    if args.copy_probe_mib:
        nbytes = args.copy_probe_mib << 20
        a = torch.empty(nbytes // 4, device="cuda")
        b = torch.empty_like(a)
        b.copy_(a)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(5):
            b.copy_(a)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / 5
        cp_gbs = 2 * nbytes / (ms / 1e3) / 1e9
        result["copy_probe"] = {"what": "runtime device-to-device copy (read + write bytes)",
                                "bytes_read": nbytes, "bytes_written": nbytes,
                                "us": ms * 1e3, "GB/s": cp_gbs, "frac_of_peak": cp_gbs / HBM_PEAK_GBS}
        # the library's own probe kernels: the commit's access pattern, read only,
        # write only and copy
        sink = torch.empty(nbytes // G.GDN_PROBE_CHUNK * 4, device="cuda")
        probes = {"read": (G.PROBE_READ, a, sink, nbytes + nbytes // 1024),
                  "write": (G.PROBE_WRITE, None, b, nbytes),
                  "copy": (G.PROBE_COPY, a, b, 2 * nbytes)}
        hp = {"what": "library probe kernels, 16-byte non-temporal pieces, 4 KiB per "
                      "workgroup instruction, XCD-contiguous ids (bytes read + written)"}
        for name, (kind, src_t, dst_t, moved) in probes.items():
            G.gdn_bandwidth_probe(kind, src_t, dst_t, nbytes)
            torch.cuda.synchronize()
            e0.record()
            for _ in range(5):
                G.gdn_bandwidth_probe(kind, src_t, dst_t, nbytes)
            e1.record()
            torch.cuda.synchronize()
            pms = e0.elapsed_time(e1) / 5
            gbs = moved / (pms / 1e3) / 1e9
            hp[name] = {"us": pms * 1e3, "GB/s": gbs, "frac_of_peak": gbs / HBM_PEAK_GBS}
        # read ceiling at the size of one verify launch: launch ramp and drain
        # weigh more at ~100 MB than at 1 GiB; the reads rotate through the
        # 1 GiB buffer so that no repetition is served from the 256 MB cache
        vb = acc["verify_bytes_per_launch"]
        vn = vb - vb % G.GDN_PROBE_CHUNK
        if 0 < vn <= nbytes:
            reps = 10
            offs = [(i * vn) % (nbytes - vn + 1) // 16 * 16 for i in range(reps)]
            views = [a.view(torch.uint8)[o:o + vn] for o in offs]
            G.gdn_bandwidth_probe(G.PROBE_READ, views[0], sink, vn)
            torch.cuda.synchronize()
            e0.record()
            for v_ in views:
                G.gdn_bandwidth_probe(G.PROBE_READ, v_, sink, vn)
            e1.record()
            torch.cuda.synchronize()
            pms = e0.elapsed_time(e1) / reps
            gbs = vn / (pms / 1e3) / 1e9
            hp["read_at_verify_launch_bytes"] = {"bytes": vn, "us": pms * 1e3, "GB/s": gbs,
                                                 "frac_of_peak": gbs / HBM_PEAK_GBS}
        result["hbm_probe"] = hp
        del a, b, sink

    if not args.no_native and not spec.ring_steps:   # the native window has no ring mode
        native_graph = capture(st.native_all)
        for _ in range(args.warmup):
            native_graph.replay()
            st.native_accept()
        torch.cuda.synchronize()
        nwall, nv_arr, na_arr = timed_loop(args.steps, native_graph.replay, st.native_accept, L)
        nv_ms, na_ms = float(np.mean(nv_arr)) / L, float(np.mean(na_arr))
        result["native_baseline"] = {
            "what": "same verify arithmetic writing the state after every draft token, "
                    "then one all-layer copy of the accepted state",
            "ms_per_step": nwall, "value": updates / (nwall / 1e3), "unit": "state-updates/s",
            "window_us_per_launch": nv_ms * 1e3,
            "window_GB/s": acc["native_bytes_per_launch"] / (nv_ms / 1e3) / 1e9,
            "accept_us": na_ms * 1e3,
            "accept_GB/s": acc["accept_bytes_per_launch"] / (na_ms / 1e3) / 1e9,
            "speedup_of_replay": nwall / wall,
        }
        log(f"native: step {nwall:.3f} ms (window {nv_ms * 1e3:.1f} us/layer, accept {na_ms * 1e3:.1f} us)")
        st.snaps = None
        del native_graph

    if not args.no_cpu:
        log("timing the CPU oracle on one full step ...")
        result["cpu_baseline"] = cpu_baseline(wl, acc, a_ch=st.a_ch)

    if not args.no_all_configs:
        del st, wl
        torch.cuda.empty_cache()
        log("every workload, the same step timing ...")
        result["all_configs"] = all_configs(args.steps, args.warmup)
        _PROBE_BUF.clear()
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
