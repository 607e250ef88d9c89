"""Seeded synthetic workloads for the verify / commit path.

This module only draws inputs. It holds none of the method's arithmetic, and
both the GPU path and the CPU oracle take their inputs from it. Integer
structure (accepted counts, slots, offsets) comes from ``numpy.random
.default_rng(seed)`` on the host; float tensors come from a
``torch.Generator`` seeded with the same seed on the target device. The draws
are therefore deterministic per (workload, seed, device); CPU and GPU draws of
the same workload differ, so tests always hand the oracle host copies of the
exact device inputs.

Value distributions (the same for every workload):
  * checkpoint state S ~ N(0, 0.05^2), fp32 (a bf16 pool holds the RNE cast);
  * q, k ~ N(0, 1), L2-normalised in fp32, stored as bf16;  v ~ N(0, 1), bf16;
  * log-gate a = -softplus(N(0, 1)) and write strength beta = sigmoid(N(0, 1)),
    both fp32 (the gate the method multiplies by is exp(a), in (0, 1]).

Layouts produced (K = V = 128 unless a test shrinks them):
  * ``state``: one tensor [L][slots][HV][V][K]; layer l is ``state[l]``;
  * ``qkv``: the packed short-conv output, [L][tokens][(2*HK + HV)*K] bf16; q,
    k and v are strided views into it (token stride (2*HK + HV)*K);
  * ``a``, ``beta``: [L][tokens][HV] fp32;
  * row arrays, int32 [B]: ``state_slot`` (-1 = null), ``rec_slot``,
    ``tok_start``, ``win_len`` (0 = padding), ``n_accept``;
  * ring + align workloads add ``p0`` (tokens already folded into the
    checkpoint), ``block_table`` [B][cols] (-1 = unallocated) and ``block``.

The five workloads follow the pages' shapes: 128x128 fp32 heads, MTP with 4
verify tokens, a 16-token replay ring and 64-token blocks (lmdeploy PR #5028,
Performance test settings), graph-padding rows with a null slot and a zero
window (vLLM RecoverSSM PR, Purpose).
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace

import numpy as np
import torch


@dataclass(frozen=True)
class WorkloadSpec:
    name: str
    layers: int
    rows: int                 # B, including padding rows
    hv: int
    hk: int
    window: int               # verify tokens per real row per step (D)
    rec_tokens: int           # record capacity per row (T)
    n_lo: int                 # accepted count ~ U{n_lo .. n_hi}
    n_hi: int
    num_slots: int
    slot_mode: str = "contiguous"   # or "random": distinct random slots
    pad_rows: int = 0         # graph-padding rows, placed at the tail
    ring_steps: int = 0       # >0: target-only ring, one token per step
    block: int = 0            # >0: align mode with this block size
    dk: int = 128
    dv: int = 128
    seed: int = 1000
    description: str = ""


TINY = WorkloadSpec(
    "tiny_l1_b1_h1", layers=1, rows=1, hv=1, hk=1, window=4, rec_tokens=4,
    n_lo=0, n_hi=4, num_slots=1, seed=1000,
    description="1 layer, 1 sequence, 1 head, D=4; accepted n swept 0..4")
SINGLE_LAYER = WorkloadSpec(
    "single_layer_b16_hv16_hk8", layers=1, rows=16, hv=16, hk=8, window=4, rec_tokens=4,
    n_lo=1, n_hi=4, num_slots=16, seed=1001,
    description="1 layer, batch 16, 16 value / 8 key heads, D=4, n~U{1..4}, contiguous slots")
ALL_LAYER = WorkloadSpec(
    "all_layer_commit_l36_b16", layers=36, rows=16, hv=32, hk=16, window=4, rec_tokens=4,
    n_lo=1, n_hi=4, num_slots=64, slot_mode="random", seed=1002,
    description="36 layers, batch 16, 32/16 heads, D=4, n~U{1..4}, 64-slot pool, random slots")
MTP_B64 = WorkloadSpec(
    "mtp_decode_l48_b64_d4", layers=48, rows=64, hv=32, hk=16, window=4, rec_tokens=4,
    n_lo=0, n_hi=4, num_slots=128, slot_mode="random", pad_rows=6, seed=1003,
    description="48 layers, batch 64 (58 real + 6 graph-padding rows), 32/16 heads, D=4, "
                "n~U{0..4}, 128-slot pool")
RING_ALIGN = WorkloadSpec(
    "ring_align_l36_b256_l16", layers=36, rows=256, hv=32, hk=16, window=1, rec_tokens=16,
    n_lo=16, n_hi=16, num_slots=576, slot_mode="random", ring_steps=16, block=64, seed=1004,
    description="36 layers, batch 256, 32/16 heads, one token per step, 16-step replay ring "
                "flushed by one align-mode commit, 64-token blocks")

WORKLOADS = {s.name: s for s in (TINY, SINGLE_LAYER, ALL_LAYER, MTP_B64, RING_ALIGN)}
ORDERED = [TINY, SINGLE_LAYER, ALL_LAYER, MTP_B64, RING_ALIGN]


@dataclass
class Workload:
    spec: WorkloadSpec
    state_dtype: torch.dtype
    state: torch.Tensor           # [L][slots][HV][V][K]
    qkv: torch.Tensor             # [L][tokens][(2HK+HV)*K] bf16
    a: torch.Tensor               # [L][tokens][HV] fp32
    beta: torch.Tensor            # [L][tokens][HV] fp32
    state_slot: np.ndarray
    rec_slot: np.ndarray
    tok_start: np.ndarray
    win_len: np.ndarray
    n_accept: np.ndarray
    p0: np.ndarray | None = None
    block_table: np.ndarray | None = None
    extra: dict = field(default_factory=dict)

    @property
    def tokens(self) -> int:
        return self.qkv.shape[1]

    @property
    def tokens_per_step(self) -> int:
        s = self.spec
        return s.rows if s.ring_steps else self.tokens

    def q(self, layer: int) -> torch.Tensor:
        s = self.spec
        return self.qkv[layer, :, : s.hk * s.dk].view(-1, s.hk, s.dk)

    def k(self, layer: int) -> torch.Tensor:
        s = self.spec
        return self.qkv[layer, :, s.hk * s.dk: 2 * s.hk * s.dk].view(-1, s.hk, s.dk)

    def v(self, layer: int) -> torch.Tensor:
        s = self.spec
        return self.qkv[layer, :, 2 * s.hk * s.dk:].view(-1, s.hv, s.dv)


def shrink(spec: WorkloadSpec, **kw) -> WorkloadSpec:
    """A copy of ``spec`` with some fields replaced (smaller CPU-sized cases)."""
    return replace(spec, **kw)


def _normal(shape, gen, device, std=1.0):
    return torch.randn(shape, generator=gen, device=device, dtype=torch.float32) * std


def make_workload(spec: WorkloadSpec, device="cpu", state_dtype=torch.float32,
                  seed: int | None = None) -> Workload:
    """Draw one workload. Draw order: S, q, k, v, a, beta (layer by layer), then
    the host-side integers: accepted counts, slots, padding, offsets."""
    seed = spec.seed if seed is None else seed
    dev = torch.device(device)
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    rng = np.random.default_rng(seed)

    L, B, HV, HK, K, V = spec.layers, spec.rows, spec.hv, spec.hk, spec.dk, spec.dv
    steps = max(spec.ring_steps, 1)
    tok_per_step = B if spec.ring_steps else B * spec.window
    tokens = steps * tok_per_step
    width = (2 * HK) * K + HV * V

    state = torch.empty((L, spec.num_slots, HV, V, K), dtype=state_dtype, device=dev)
    for layer in range(L):
        for s0 in range(0, spec.num_slots, 64):      # bounded temporaries
            s1 = min(spec.num_slots, s0 + 64)
            state[layer, s0:s1] = _normal((s1 - s0, HV, V, K), gen, dev, 0.05).to(state_dtype)

    qkv = torch.empty((L, tokens, width), dtype=torch.bfloat16, device=dev)
    a = torch.empty((L, tokens, HV), dtype=torch.float32, device=dev)
    beta = torch.empty((L, tokens, HV), dtype=torch.float32, device=dev)
    for layer in range(L):
        q = torch.nn.functional.normalize(_normal((tokens, HK, K), gen, dev), dim=-1)
        k = torch.nn.functional.normalize(_normal((tokens, HK, K), gen, dev), dim=-1)
        v = _normal((tokens, HV, V), gen, dev)
        qkv[layer, :, : HK * K] = q.reshape(tokens, -1).to(torch.bfloat16)
        qkv[layer, :, HK * K: 2 * HK * K] = k.reshape(tokens, -1).to(torch.bfloat16)
        qkv[layer, :, 2 * HK * K:] = v.reshape(tokens, -1).to(torch.bfloat16)
        a[layer] = -torch.nn.functional.softplus(_normal((tokens, HV), gen, dev))
        beta[layer] = torch.sigmoid(_normal((tokens, HV), gen, dev))

    n_accept = rng.integers(spec.n_lo, spec.n_hi + 1, size=B).astype(np.int32)
    if spec.slot_mode == "random":
        state_slot = rng.permutation(spec.num_slots)[:B].astype(np.int32)
    else:
        state_slot = np.arange(B, dtype=np.int32) % spec.num_slots
    rec_slot = np.arange(B, dtype=np.int32)
    win_len = np.full(B, 1 if spec.ring_steps else spec.window, np.int32)
    if spec.ring_steps:
        tok_start = np.arange(B, dtype=np.int32)          # within one step's tokens
    else:
        tok_start = (np.arange(B) * spec.window).astype(np.int32)
    if spec.pad_rows:
        pad = np.arange(B - spec.pad_rows, B)
        state_slot[pad] = -1
        win_len[pad] = 0
        n_accept[pad] = 0
        rec_slot[pad] = -1

    wl = Workload(spec, state_dtype, state, qkv, a, beta, state_slot, rec_slot, tok_start,
                  win_len, n_accept)

    if spec.block:
        assert spec.slot_mode == "random" and spec.num_slots >= 2 * B
        blk = spec.block
        m = rng.integers(256, 288, size=B)           # ~16k-token contexts, 64-token blocks
        r = rng.integers(0, blk, size=B)
        forced = [blk - spec.ring_steps, 0, blk - spec.ring_steps + 1, blk - 1]
        for i, rv in enumerate(forced):              # >= 4 rows of each special offset
            r[i * 4: i * 4 + 4] = rv
        rng.shuffle(r)
        p0 = (m * blk + r).astype(np.int32)
        c0 = (p0 - 1) // blk                          # the checkpoint's block column
        cols = int(c0.max()) + 2                      # room for the next block of every row
        slots = rng.permutation(spec.num_slots)[: 2 * B].astype(np.int32).reshape(B, 2)
        table = np.full((B, cols), -1, np.int32)
        table[np.arange(B), c0] = slots[:, 0]
        table[np.arange(B), c0 + 1] = slots[:, 1]
        wl.p0 = p0
        wl.block_table = table
        wl.state_slot = slots[:, 0].copy()            # verify reads the checkpoint's block
        wl.extra["slots"] = slots
    return wl


@dataclass
class RawGates:
    """Raw per-token gate projections of every layer and the per-head gate
    parameters, for the raw-input gating variant of verify."""
    a: torch.Tensor        # [L][tokens][HV] fp32
    b: torch.Tensor        # [L][tokens][HV] fp32
    A_log: torch.Tensor    # [L][HV] fp32
    dt_bias: torch.Tensor  # [L][HV] fp32


RAW_GATE_SEED_OFFSET = 7919


def make_raw_gates(wl: Workload, device="cpu", seed: int | None = None) -> RawGates:
    """Draw raw gate inputs for a workload from a stream of their own (the
    workload's own draws are unchanged). a, b ~ N(0, 1); per head, A_log =
    log A with A ~ U(1, 16) and dt_bias the inverse softplus of a time step
    drawn log-uniform in [1e-3, 1e-1] (the initialisation recipe of Mamba-2
    style decay parameters)."""
    s = wl.spec
    seed = (s.seed if seed is None else seed) + RAW_GATE_SEED_OFFSET
    rng = np.random.default_rng(seed)
    L, T, HV = s.layers, wl.tokens, s.hv
    a = rng.standard_normal((L, T, HV)).astype(np.float32)
    b = rng.standard_normal((L, T, HV)).astype(np.float32)
    A_log = np.log(rng.uniform(1.0, 16.0, (L, HV))).astype(np.float32)
    dt = np.exp(rng.uniform(np.log(1e-3), np.log(1e-1), (L, HV)))
    dt_bias = (dt + np.log(-np.expm1(-dt))).astype(np.float32)
    dev = torch.device(device)
    return RawGates(*(torch.as_tensor(x, device=dev) for x in (a, b, A_log, dt_bias)))


CHANNEL_DECAY_SEED_OFFSET = 65537


def make_channel_decays(wl: Workload, device="cpu", seed: int | None = None) -> torch.Tensor:
    """One log-decay per (layer, token, value head, key channel), fp32
    [L][tokens][HV][128], drawn like the scalar log-gate (-softplus of a
    standard normal) from a stream of its own."""
    s = wl.spec
    seed = (s.seed if seed is None else seed) + CHANNEL_DECAY_SEED_OFFSET
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((s.layers, wl.tokens, s.hv, 128), dtype=np.float32)
    a = -np.logaddexp(np.float32(0), x).astype(np.float32)
    return torch.as_tensor(a, device=torch.device(device))


@dataclass
class ConvInputs:
    """Short-conv state pools of every layer and the step's conv inputs."""
    state: torch.Tensor    # [L][slots][state_len][C]
    x: torch.Tensor        # [L][tokens][C]


CONV_SEED_OFFSET = 104729


def make_conv(wl: Workload, state_len: int = 3, dtype=torch.bfloat16, device="cpu",
              seed: int | None = None, channels: int | None = None) -> ConvInputs:
    """Draw short-conv states and inputs for a workload from a stream of their
    own: C = (2 HK + HV) * 128 channels by default (the mixed q/k/v a GDN
    layer's short conv runs over), values N(0, 1); state_len = (kernel width
    - 1) * dilation, 3 for a width-4 conv."""
    s = wl.spec
    seed = (s.seed if seed is None else seed) + CONV_SEED_OFFSET
    C = (2 * s.hk + s.hv) * 128 if channels is None else channels
    dev = torch.device(device)
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    state = torch.empty((s.layers, s.num_slots, state_len, C), dtype=dtype, device=dev)
    x = torch.empty((s.layers, wl.tokens, C), dtype=dtype, device=dev)
    for layer in range(s.layers):
        state[layer] = _normal((s.num_slots, state_len, C), gen, dev).to(dtype)
        x[layer] = _normal((wl.tokens, C), gen, dev).to(dtype)
    return ConvInputs(state, x)


# Per-position draft acceptance for MTP with five draft tokens, as quoted in the
# review thread of the vLLM RecoverSSM PR (position i accepted, given 0..i-1 were).
MTP_ACCEPTANCE_RATES = (0.856, 0.694, 0.558, 0.457, 0.376)
ACCEPT_SEED_OFFSET = 7919


def acceptance_rate_counts(rng: np.random.Generator, rows: int,
                           rates=MTP_ACCEPTANCE_RATES) -> np.ndarray:
    """Accepted counts drawn from per-position acceptance rates (a draft token
    at position i is accepted with probability rates[i], given the ones before
    it were), the bonus token always committed. The default rates are the
    per-position acceptance quoted for MTP K=5 in the vLLM RecoverSSM PR's
    review thread."""
    n = np.ones(rows, np.int32)
    alive = np.ones(rows, bool)
    prev = 1.0
    for p in rates:
        cond = p / prev
        prev = p
        acc = rng.random(rows) < cond
        alive &= acc
        n += alive
    return n


def draw_acceptance_rate_counts(wl: Workload, seed: int | None = None) -> None:
    """Replace the accepted counts of the workload's real rows (in place) by
    counts drawn from the per-position acceptance rates of its draft tokens
    (window - 1 drafts and the bonus token, so n in 1 .. window); padding rows
    keep n = 0. Not defined for the replay ring, whose flush commits every
    ring record."""
    s = wl.spec
    if s.ring_steps:
        raise ValueError("the replay ring commits all of its records at the flush")
    if s.window - 1 > len(MTP_ACCEPTANCE_RATES):
        raise ValueError(f"acceptance rates are given for {len(MTP_ACCEPTANCE_RATES)} drafts")
    rng = np.random.default_rng((s.seed if seed is None else seed) + ACCEPT_SEED_OFFSET)
    real = np.flatnonzero(wl.win_len > 0)
    wl.n_accept[real] = acceptance_rate_counts(rng, len(real), MTP_ACCEPTANCE_RATES[: s.window - 1])
