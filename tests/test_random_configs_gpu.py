"""GPU parity over seeded random configurations: layer count, rows, value and
key head counts (group sizes 1 to 3), record capacity T from 1 to 16 (so
every compiled window capacity and both verify launch shapes), output scale,
state dtype, null rows, and per-row windows that start after a per-row
number of pending ring records (each row's T-token window verified in two
launches: positions 0..j-1, then j..j+w-1 with ring base j). The commit then
takes a random accepted count per row, in place or into another slot, with an
align-mode boundary for some rows (into a spare slot or into the source
slot). Every output, record, final and boundary state is checked against the
oracle's native rule over the row's j + w tokens (the bars of
test_parity_gpu), everything outside the write sets is checked unchanged
(checkpoints, other slots, other tokens' outputs, unused record positions).

A second set draws the same kind of configurations for verify's options:
gates formed in the kernel from raw projections, outputs rounded to bf16, and
one decay per key channel (the per-channel record kind, replayed column by
column), with the oracle's matching rule."""
import types

import numpy as np
import pytest
import torch

import oracle
import oracle_pool as OP
import gated_deltanet_speculative_gdn_amd as G
from gated_deltanet_speculative_gdn_amd import workloads as W
from gpu_harness import dev_i32
from test_parity_gpu import (TOL, assert_bitwise, assert_close, assert_close_blocks,
                             assert_close_elementwise, assert_fp64_accuracy, check_bf16,
                             pool_bits)

pytestmark = pytest.mark.gpu

NAN = float("nan")


def draw_case(seed):
    rng = np.random.default_rng(7000 + seed)
    c = types.SimpleNamespace()
    c.dtype = (torch.float32, torch.bfloat16)[seed % 2]
    c.L = int(rng.integers(1, 3))
    c.hk = int(rng.choice([1, 2, 4]))
    c.hv = c.hk * int(rng.choice([1, 2, 3]))
    c.T = int(rng.choice([1, 2, 3, 4, 4, 4, 5, 7, 8, 11, 16]))   # MTP-sized windows weighted
    c.B = int(rng.integers(1, 13))
    c.scale = float(rng.choice([1.0, 128 ** -0.5]))
    B, T = c.B, c.T
    c.null = rng.random(B) < 0.15
    c.j = rng.integers(0, T, size=B).astype(np.int32)              # pending records
    c.w = np.array([rng.integers(0, T - j + 1) for j in c.j], np.int32)
    c.tot = c.j + c.w
    c.n = np.array([rng.integers(0, t + 1) for t in c.tot], np.int32)
    c.in_place = rng.random(B) < 0.5
    c.bl = np.array([rng.integers(1, n) if n >= 2 and rng.random() < 0.5 else 0 for n in c.n],
                    np.int32)
    c.b_src = rng.random(B) < 0.5                                   # boundary into the source
    return c


def assert_bf16_close(got, ref, mask, what):
    """Elementwise within one bf16 ulp of the fp32 reference plus the fp32
    tolerance of the vector's largest value, on the vectors ``mask`` selects."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    mag = np.abs(ref)
    ulp = np.exp2(np.floor(np.log2(np.where(mag > 0, mag, 1e-38))) - 7)
    slack = TOL * mag.max(axis=-1, keepdims=True)
    bad = (np.abs(got - ref) > ulp + slack) & np.asarray(mask)[..., None]
    assert not bad.any(), f"{what}: {int(bad.sum())} elements more than one bf16 ulp off"


def run_case(seed, kind="scalar", out_bf16=False):
    """kind: "scalar" (log-gates and write strengths as inputs), "raw" (gates
    formed in the kernel) or "channel" (one log-decay per key channel)."""
    c = draw_case(seed)
    L, B, HV, HK, T = c.L, c.B, c.hv, c.hk, c.T
    spec = W.shrink(W.SINGLE_LAYER, layers=L, rows=B, hv=HV, hk=HK, window=T, rec_tokens=T,
                    n_lo=0, n_hi=0, num_slots=3 * B + 2, slot_mode="random", pad_rows=0)
    wl = W.make_workload(spec, device="cuda", state_dtype=c.dtype, seed=7000 + seed)
    print(f"case {seed} {kind}{' bf16-out' if out_bf16 else ''}: L={L} B={B} HV={HV} HK={HK} "
          f"T={T} dtype={c.dtype} scale={c.scale:.4f} j={c.j.tolist()} w={c.w.tolist()} "
          f"n={c.n.tolist()} bl={c.bl.tolist()}", flush=True)
    channel = kind == "channel"
    record_kind = G.RECORD_CHANNEL if channel else G.RECORD_CORRECTION
    rg = W.make_raw_gates(wl, device="cuda") if kind == "raw" else None
    a_ch = W.make_channel_decays(wl, device="cuda") if channel else None

    slot = np.where(c.null, -1, wl.state_slot).astype(np.int32)
    spare = iter(np.setdiff1d(np.arange(spec.num_slots), wl.state_slot).tolist())
    dst = np.array([s if (ip or s < 0) else next(spare) for s, ip in zip(slot, c.in_place)],
                   np.int32)
    bs = np.full(B, -1, np.int32)
    for b in range(B):
        if c.bl[b] > 0:
            bs[b] = slot[b] if (c.b_src[b] and dst[b] != slot[b]) else next(spare)
    bl = np.where(bs >= 0, c.bl, 0).astype(np.int32)

    rec = G.Pools.alloc_records(L, B, HV, T, record_kind=record_kind)
    rec.fill_(NAN)
    pools = G.Pools(wl.state, rec, HK, T, record_kind)
    out = torch.full((L, wl.tokens, HV, 128), NAN, device="cuda",
                     dtype=torch.bfloat16 if out_bf16 else torch.float32)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    pre = wl.state.clone()
    rec_slot = dev_i32(np.arange(B))
    base_tok = (np.arange(B) * T).astype(np.int32)

    # two verify launches per layer: the pending prefix, then the window after it
    for layer in range(L):
        if kind == "raw":
            a_in, b_in, gk = rg.a[layer], rg.b[layer], dict(A_log=rg.A_log[layer],
                                                            dt_bias=rg.dt_bias[layer])
        else:
            a_in = a_ch[layer] if channel else wl.a[layer]
            b_in, gk = wl.beta[layer], {}
        for ts, win, base in ((base_tok, c.j, np.zeros(B, np.int32)), (base_tok + c.j, c.w, c.j)):
            G.gdn_verify(pools, layer, dev_i32(slot), rec_slot, dev_i32(ts), dev_i32(win),
                         dev_i32(base), wl.q(layer), wl.k(layer), wl.v(layer), a_in, b_in,
                         out[layer], scale=c.scale, err_flags=err, **gk)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    assert torch.equal(pool_bits(wl.state), pool_bits(pre)), "verify wrote a checkpoint"

    G.gdn_commit_all_layers(pools, dev_i32(slot), dev_i32(dst), rec_slot, dev_i32(c.n),
                            dev_i32(bl), dev_i32(bs), err_flags=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0

    live = (slot >= 0) & (c.tot > 0)
    written = set()
    for b in range(B):
        if slot[b] >= 0 and c.n[b] > 0:
            written.add(int(dst[b]))
            if bl[b] > 0 and bs[b] != dst[b]:
                written.add(int(bs[b]))
    for layer in range(L):
        keep = [s for s in range(spec.num_slots) if s not in written]
        idx = torch.as_tensor(keep, device="cuda")
        assert torch.equal(pool_bits(wl.state[layer].index_select(0, idx)),
                           pool_bits(pre[layer].index_select(0, idx))), "slot outside the plan"

    # nothing written outside the windows: outputs of other tokens, record positions >= j + w
    tok_written = np.zeros(wl.tokens, bool)
    for b in np.nonzero(live)[0]:
        tok_written[base_tok[b]: base_tok[b] + c.tot[b]] = True
    o_all = out.float().cpu().numpy()
    assert np.isnan(o_all[:, ~tok_written]).all(), "an output outside the windows was written"
    assert not np.isnan(o_all[:, tok_written]).any()
    r_all = rec.cpu().numpy()
    fields = 3 if channel else 2                  # [T][128] fields before the gates (if any)
    for b in range(B):
        blk = r_all[:, b].reshape(L, HV, -1)
        t_used = int(c.tot[b]) if live[b] else 0
        for part in range(fields):
            seg = blk[..., part * T * 128: (part + 1) * T * 128].reshape(L, HV, T, 128)
            assert np.isnan(seg[:, :, t_used:]).all(), f"row {b}: record past its window"
        if not channel:
            gseg = blk[..., 2 * T * 128: 2 * T * 128 + T]
            assert np.isnan(gseg[:, :, t_used:]).all(), f"row {b}: gate past its window"

    rows = np.nonzero(live)[0]
    if rows.size == 0:
        return
    R = rows.size
    tok = base_tok[rows][:, None] + np.arange(T)[None, :]
    tix = torch.as_tensor(tok.reshape(-1).astype(np.int64), device="cuda")
    tot = c.tot[rows]
    n = c.n[rows]
    keep = np.stack([n, np.where(bl[rows] > 0, bl[rows], -1)], 1).astype(np.int32)
    keep_h = np.repeat(keep, HV, axis=0)
    valid = np.repeat(np.arange(T)[None, :] < tot[:, None], HV, axis=0)
    vm = valid[..., None]
    shim = types.SimpleNamespace(wl=wl)
    for layer in range(L):
        S0 = OP.to_f32(pre[layer].index_select(
            0, torch.as_tensor(slot[rows].astype(np.int64), device="cuda"))).reshape(R * HV, 128, 128)
        g = OP.gather_tokens(wl, layer, tok, tot, S0)
        if kind == "raw":                 # the oracle's gates from the same raw inputs
            lg, be = oracle.raw_gates(rg.a[layer].cpu().numpy(), rg.b[layer].cpu().numpy(),
                                      rg.A_log[layer].cpu().numpy(),
                                      rg.dt_bias[layer].cpu().numpy())
            g["a"] = np.ascontiguousarray(lg[tok].transpose(0, 2, 1)).reshape(R * HV, T)
            g["beta"] = np.ascontiguousarray(be[tok].transpose(0, 2, 1)).reshape(R * HV, T)
        if channel:
            ach = OP.to_f32(a_ch[layer].index_select(0, tix)).reshape(R, T, HV, 128)
            g["a"] = np.ascontiguousarray(ach.transpose(0, 2, 1, 3)).reshape(R * HV, T, 128)
        args = (g["S0"], g["w"], g["q"], g["k"], g["v"], g["a"], g["beta"])
        rule = oracle.native_heads_ch if channel else oracle.native_heads
        res = rule(*args, scale=c.scale, keep=keep_h)
        r64 = rule(*args, scale=c.scale, keep=keep_h, dtype=np.float64)
        o = out[layer].index_select(0, tix).float().reshape(R, T, HV, 128).permute(0, 2, 1, 3)
        o = np.where(vm, o.reshape(R * HV, T, 128).cpu().numpy(), 0)
        if out_bf16:
            assert_bf16_close(o, res.o, valid, f"layer {layer} bf16 outputs")
        else:
            assert_close(o, np.where(vm, res.o, 0), f"layer {layer} outputs")
            assert_fp64_accuracy(o, res.o, r64.o, f"layer {layer} output vectors", mask=valid)
        blk = r_all[layer, rows].reshape(R * HV, -1)
        d = np.where(vm, blk[:, : T * 128].reshape(-1, T, 128), 0)
        kh = np.where(vm, blk[:, T * 128: 2 * T * 128].reshape(-1, T, 128), 0)
        assert_close_blocks(d, np.where(vm, res.rec_delta, 0), 1,
                            f"layer {layer} correction vectors")
        assert_fp64_accuracy(d, res.rec_delta, r64.rec_delta, f"layer {layer} correction vectors",
                             mask=valid)
        assert_close_blocks(kh, np.where(vm, res.rec_khat, 0), 1, f"layer {layer} key vectors")
        if channel:
            gg = np.where(vm, blk[:, 2 * T * 128: 3 * T * 128].reshape(-1, T, 128), 0)
            assert_close_elementwise(gg, np.where(vm, res.rec_alpha, 0), f"layer {layer} decays")
        else:
            gg = np.where(valid, blk[:, 2 * T * 128: 2 * T * 128 + T], 0)
            assert_close_elementwise(gg, np.where(valid, res.rec_g, 0), f"layer {layer} gates")
        d32, k32, g32 = (x.astype(np.float32) for x in (d, kh, gg))
        replay = oracle.replay_heads_ch if channel else oracle.replay_heads
        for which, cnt, slots_of in ((0, n, dst[rows]), (1, bl[rows], bs[rows])):
            sel = (cnt > 0) if which == 0 else (cnt > 0) & (bs[rows] != dst[rows])
            if not sel.any():
                continue
            sel_h = np.repeat(sel, HV)
            rep = replay(g["S0"][sel_h], np.repeat(cnt[sel], HV), d32[sel_h], k32[sel_h],
                         g32[sel_h])
            what = ("final", "boundary")[which]
            if c.dtype == torch.float32:
                got = OP.to_f32(wl.state[layer].index_select(
                    0, torch.as_tensor(slots_of[sel].astype(np.int64), device="cuda")))
                got = got.reshape(-1, 128, 128)
                assert_close_blocks(got, res.kept[sel_h, which], 2, f"layer {layer} {what} heads")
                assert_bitwise(got, rep, f"layer {layer} {what} vs replay of GPU records")
            else:
                check_bf16(shim, layer, slots_of[sel], rep, res.kept[sel_h, which], what)


@pytest.mark.parametrize("seed", range(20))
def test_random_configuration(gdn, seed):
    run_case(seed)


VARIANTS = [("raw", False), ("scalar", True), ("channel", False), ("raw", True)]


@pytest.mark.parametrize("seed", range(20, 32))
def test_random_configuration_variants(gdn, seed):
    kind, out_bf16 = VARIANTS[seed % len(VARIANTS)]
    run_case(seed, kind, out_bf16)
