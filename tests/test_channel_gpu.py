"""GPU parity of the per-key-channel decay variant (a reading of Kimi-K3 KDA,
which the vLLM RecoverSSM PR's Purpose names as a user of the same
record-and-replay protocol without its arithmetic; here the scalar decay
becomes one decay per key channel, the record keeps alpha[K], and the commit
replays h[v][k] = fma(delta[v], k_hat[k], h[v][k] * alpha[k])).

Bars as the other parity tests: outputs, records and committed states within
the normwise 1e-5 of the oracle's per-channel rule; the commit bit-exact
against the oracle's replay of the GPU's own records (bf16 pools: RNE of it,
and within one bf16 ulp of the fp32 native states); the native snapshot path
bit-identical to verify and commit; ring mode against the oracle over all 16
ring tokens."""
import numpy as np
import pytest
import torch

import oracle
import oracle_pool as OP
import gated_deltanet_speculative_gdn_amd as G
from gated_deltanet_speculative_gdn_amd import workloads as W
from gpu_harness import Harness, dev_i32
from test_parity_gpu import (TOL, assert_bitwise, assert_close, assert_close_blocks,
                             assert_close_elementwise, assert_fp64_accuracy, check_bf16,
                             pool_bits)

pytestmark = pytest.mark.gpu


def channel_records(h, layer, rows):
    """(delta [R*HV][T][V], k_hat [R*HV][T][K], alpha [R*HV][T][K]) of the rows."""
    s = h.s
    T = s.rec_tokens
    rs = torch.as_tensor(h.wl.rec_slot[np.asarray(rows)].astype(np.int64), device="cuda")
    blk = h.rec[layer].index_select(0, rs).reshape(len(rows) * s.hv, -1).cpu().numpy()
    return (blk[:, : T * 128].reshape(-1, T, 128), blk[:, T * 128: 2 * T * 128].reshape(-1, T, 128),
            blk[:, 2 * T * 128: 3 * T * 128].reshape(-1, T, 128))


def verify_ch(h, a_ch, layer, *, step=None, out=None, rec_base=None):
    wl, s = h.wl, h.s
    sl = slice(step * s.rows, (step + 1) * s.rows) if step is not None else slice(0, wl.tokens)
    G.gdn_verify(h.pools, layer, h.state_slot, h.rec_slot, h.tok_start, h.win_len, rec_base,
                 wl.q(layer)[sl], wl.k(layer)[sl], wl.v(layer)[sl], a_ch[layer, sl],
                 wl.beta[layer, sl], h.out[layer, sl] if out is None else out, err_flags=h.err)


def check_channel_layer(h, a_ch, layer, rows, n, pre_state, *, T=None, bnd=None, dst=None):
    wl, s = h.wl, h.s
    rows = np.asarray(rows)
    keep = [np.asarray(n)]
    if bnd is not None:
        keep.append(np.where(bnd[0] > 0, bnd[0], -1))
    g, res = OP.run_layer_ch(wl, a_ch, layer, rows, keep=np.stack(keep, 1), T=T, state=pre_state)
    res64 = oracle.native_heads_ch(g["S0"], g["w"], g["q"], g["k"], g["v"], g["a"], g["beta"],
                                   dtype=np.float64)
    Tw = g["q"].shape[1]
    valid = np.arange(Tw)[None, :] < g["w"][:, None]
    o = np.where(valid[..., None], h.outputs(layer, rows, T), 0)
    assert_close(o, np.where(valid[..., None], res.o, 0), f"layer {layer} outputs")
    assert_fp64_accuracy(o, res.o, res64.o, f"layer {layer} output vectors", mask=valid)
    d, kh, al = (x[:, :Tw] for x in channel_records(h, layer, rows))
    d, kh, al = (np.where(valid[..., None], x, 0).astype(np.float32) for x in (d, kh, al))
    assert_close_blocks(d, res.rec_delta, 1, f"layer {layer} correction vectors")
    assert_fp64_accuracy(d, res.rec_delta, res64.rec_delta, f"layer {layer} correction vectors",
                         mask=valid)
    assert_close_blocks(kh, res.rec_khat, 1, f"layer {layer} key vectors")
    assert_close_elementwise(al, res.rec_alpha, f"layer {layer} decays")
    n = np.asarray(n)
    dst = wl.state_slot[rows] if dst is None else np.asarray(dst)
    live = n > 0
    # (rows selected, their slots, replayed counts per head, oracle states, name)
    targets = [(live, dst[live], np.repeat(n[live], s.hv), res.kept[np.repeat(live, s.hv), 0],
                "final")]
    if bnd is not None and (bnd[0] > 0).any():
        has = bnd[0] > 0
        targets.append((has, bnd[1][has], np.repeat(bnd[0][has], s.hv),
                        res.kept[np.repeat(has, s.hv), 1], "boundary"))
    for sel_rows, slots, nn, ref, what in targets:
        sel = np.repeat(sel_rows, s.hv)
        rep = oracle.replay_heads_ch(g["S0"][sel], nn, d[sel], kh[sel], al[sel])
        if wl.state_dtype == torch.float32:
            got = h.heads(layer, slots)
            assert_close_blocks(got, ref, 2, f"layer {layer} {what} state heads")
            assert_bitwise(got, rep, f"layer {layer} {what} vs replay of GPU records")
        else:
            check_bf16(h, layer, slots, rep, ref, what)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["fp32", "bf16"])
def test_channel_verify_and_commit(gdn, dtype):
    spec = W.shrink(W.ALL_LAYER, layers=3)
    wl = W.make_workload(spec, device="cuda", state_dtype=dtype)
    a_ch = W.make_channel_decays(wl, device="cuda")
    h = Harness(wl, record_kind=G.RECORD_CHANNEL)
    pre = wl.state.clone()
    for layer in range(spec.layers):
        verify_ch(h, a_ch, layer)
    torch.cuda.synchronize()
    assert torch.equal(pool_bits(wl.state), pool_bits(pre)), "verify wrote the checkpoint"
    h.commit()
    torch.cuda.synchronize()
    assert h.err_value() == 0
    for layer in range(spec.layers):
        check_channel_layer(h, a_ch, layer, np.arange(spec.rows), wl.n_accept, pre[layer])


def test_channel_longest_windows(gdn):
    """16 records per row, every position in one window, n = 1..16."""
    T = 16
    spec = W.shrink(W.SINGLE_LAYER, rows=8, window=T, rec_tokens=T, n_lo=1, n_hi=T)
    wl = W.make_workload(spec, device="cuda", seed=121)
    a_ch = W.make_channel_decays(wl, device="cuda")
    h = Harness(wl, record_kind=G.RECORD_CHANNEL)
    pre = wl.state.clone()
    verify_ch(h, a_ch, 0)
    h.commit()
    torch.cuda.synchronize()
    assert h.err_value() == 0
    check_channel_layer(h, a_ch, 0, np.arange(spec.rows), wl.n_accept, pre[0])


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["fp32", "bf16"])
def test_channel_native_snapshots_match_verify_and_commit(gdn, dtype):
    spec = W.shrink(W.ALL_LAYER, layers=2)
    wl = W.make_workload(spec, device="cuda", state_dtype=dtype)
    a_ch = W.make_channel_decays(wl, device="cuda")
    h = Harness(wl, record_kind=G.RECORD_CHANNEL)
    for layer in range(spec.layers):
        verify_ch(h, a_ch, layer)
    out_v = h.out.clone()
    out_n = torch.full_like(h.out, float("nan"))
    snaps = [torch.empty((spec.rows, spec.hv, spec.rec_tokens, 128, 128), dtype=dtype,
                         device="cuda") for _ in range(spec.layers)]
    for layer in range(spec.layers):
        G.gdn_native_window(h.pools, layer, h.state_slot, h.tok_start, h.win_len, wl.q(layer),
                            wl.k(layer), wl.v(layer), a_ch[layer], wl.beta[layer], out_n[layer],
                            snaps[layer], err_flags=h.err)
    torch.cuda.synchronize()
    assert torch.equal(out_n.view(torch.int32), out_v.view(torch.int32))
    h.commit()
    torch.cuda.synchronize()
    for layer in range(spec.layers):
        for b in range(spec.rows):
            n = int(wl.n_accept[b])
            if n:
                got = pool_bits(wl.state[layer, int(wl.state_slot[b])])
                assert torch.equal(got, pool_bits(snaps[layer][b, :, n - 1])), (layer, b)
    assert h.err_value() == 0


def test_channel_ring_align(gdn):
    """The replay ring with per-channel decays: 16 single-token verify steps per
    layer with the pending records' corrections, keys and decays applied
    first, then one align-mode commit of the 16 tokens (boundaries into the
    source slot)."""
    spec = W.shrink(W.RING_ALIGN, layers=2, rows=32, num_slots=80, hv=4, hk=2, seed=3200)
    wl = W.make_workload(spec, device="cuda")
    a_ch = W.make_channel_decays(wl, device="cuda")
    h = Harness(wl, record_kind=G.RECORD_CHANNEL)
    pre = wl.state.clone()
    for step in range(spec.ring_steps):
        base = dev_i32(np.full(spec.rows, step))
        for layer in range(spec.layers):
            verify_ch(h, a_ch, layer, step=step, rec_base=base)
    torch.cuda.synchronize()
    assert torch.equal(pool_bits(wl.state), pool_bits(pre)), "verify wrote the checkpoint"
    src, dst, bl, bs, perr = oracle.align_plan(wl.p0, wl.n_accept, wl.block_table, spec.block,
                                               spec.rec_tokens)
    assert not perr.any() and (bl > 0).any()
    h.commit(src=dev_i32(src), dst=dev_i32(dst), n=h.n_accept, bnd_len=dev_i32(bl),
             bnd_slot=dev_i32(bs))
    torch.cuda.synchronize()
    assert h.err_value() == 0
    for layer in range(spec.layers):
        check_channel_layer(h, a_ch, layer, np.arange(spec.rows), wl.n_accept, pre[layer],
                            bnd=(bl, bs), dst=dst)


@pytest.mark.parametrize("seed", [41, 42])
def test_channel_extreme_decays(gdn, seed):
    """Channels that never decay (log-decay 0), channels decayed into the fp32
    subnormal range (-100) and channels wiped (-inf) in the same window."""
    spec = W.shrink(W.ALL_LAYER, layers=1)
    wl = W.make_workload(spec, device="cuda", seed=seed)
    a_ch = W.make_channel_decays(wl, device="cuda")
    a_ch[..., :16] = 0.0
    a_ch[..., 16:32] = -100.0
    a_ch[:, ::3, :, 32:40] = float("-inf")
    h = Harness(wl, record_kind=G.RECORD_CHANNEL)
    pre = wl.state.clone()
    verify_ch(h, a_ch, 0)
    h.commit()
    torch.cuda.synchronize()
    assert h.err_value() == 0
    check_channel_layer(h, a_ch, 0, np.arange(spec.rows), wl.n_accept, pre[0])


def test_channel_records_with_conv_compaction(gdn):
    """The fused launch with per-channel decay records: the state replay equals
    a plain commit of the same records bit for bit, and the conv states equal
    the oracle's token walk."""
    from test_conv_commit_gpu import expected_pool, raw
    spec = W.shrink(W.ALL_LAYER, layers=2)
    wl = W.make_workload(spec, device="cuda", seed=131)
    a_ch = W.make_channel_decays(wl, device="cuda")
    cv = W.make_conv(wl, state_len=3, dtype=torch.bfloat16, device="cuda")
    h = Harness(wl, record_kind=G.RECORD_CHANNEL)
    for layer in range(spec.layers):
        verify_ch(h, a_ch, layer)
    torch.cuda.synchronize()
    ref_state = wl.state.clone()
    ref_pools = G.Pools(ref_state, h.rec, spec.hk, spec.rec_tokens, G.RECORD_CHANNEL)
    G.gdn_commit_all_layers(ref_pools, h.state_slot, h.state_slot, h.rec_slot, h.n_accept,
                            err_flags=h.err)
    pre = raw(cv.state)
    x = raw(cv.x)
    G.gdn_commit_all_layers_conv(h.pools, G.ConvPools(cv.state, cv.x), h.state_slot,
                                 h.state_slot, h.rec_slot, h.n_accept,
                                 conv_tok_start=h.tok_start, err_flags=h.err)
    torch.cuda.synchronize()
    assert h.err_value() == 0
    assert torch.equal(pool_bits(wl.state), pool_bits(ref_state)), "state replay differs"
    got = raw(cv.state)
    for layer in range(spec.layers):
        exp = expected_pool(pre[layer], x[layer], range(spec.rows), wl.state_slot, wl.state_slot,
                            wl.n_accept, wl.tok_start)
        np.testing.assert_array_equal(got[layer], exp, err_msg=f"layer {layer}")
