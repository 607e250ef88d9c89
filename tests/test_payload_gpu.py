"""GPU parity of the payload-record variant (tokenspeed PR, Motivation: keep
the per-token K/V/a/b inputs and recompute the accepted transitions at commit).

Verify writes, per (token, value head), the raw bf16 key of its key head, the
raw bf16 value, the decay and the write strength; the commit normalises the
key, recomputes u = (g h) k_hat with a row reduction, the correction and the
update. Bars:
  * verify outputs bit-identical to the correction-record verify (same code);
    the record's key and value bits equal to the inputs, its decay equal to
    the correction record's decay bit for bit, its write strength equal to
    the input beta;
  * committed states within the fp32 tolerance (normwise 1e-5 per layer) of
    the oracle's native per-token states, bf16 pools within one bf16 ulp plus
    that tolerance. They are not bit-identical to the native states: the
    commit's reduction order is its own, which is the trade the correction
    record avoids.
"""
import numpy as np
import pytest
import torch

import oracle
import oracle_pool as OP
import gated_deltanet_speculative_gdn_amd as G
from gated_deltanet_speculative_gdn_amd import workloads as W
from gpu_harness import Harness, dev_i32
from test_parity_gpu import TOL, assert_bitwise, assert_close_blocks, pool_bits

pytestmark = pytest.mark.gpu


def payload_fields(h, layer, rows):
    """(k bits [R*HV][T][K] uint16, v bits [R*HV][T][V], gate [R*HV][T], beta [R*HV][T])."""
    s = h.s
    T = s.rec_tokens
    rs = torch.as_tensor(h.wl.rec_slot[np.asarray(rows)].astype(np.int64), device="cuda")
    blk = h.rec[layer].index_select(0, rs).reshape(len(rows) * s.hv, -1)
    u16 = blk.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    f32 = blk.cpu().numpy()
    k = u16[:, : T * s.dk].reshape(-1, T, s.dk)
    v = u16[:, T * s.dk: T * (s.dk + s.dv)].reshape(-1, T, s.dv)
    g = f32[:, T * 128: T * 128 + T]
    be = f32[:, T * 129: T * 129 + T]
    return k, v, g, be


def input_bits(wl, layer, rows):
    """Raw bf16 bits of each (row, value head)'s key (its key head) and value
    over the row's window: [R*HV][T][128] each."""
    s = wl.spec
    tok = OP.token_index(wl, rows)
    tix = torch.as_tensor(tok.reshape(-1).astype(np.int64), device="cuda")
    hk_of = np.arange(s.hv) // (s.hv // s.hk)
    kb = wl.k(layer).index_select(0, tix).contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    vb = wl.v(layer).index_select(0, tix).contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    R, T = len(rows), tok.shape[1]
    kb = kb.reshape(R, T, s.hk, 128)[:, :, hk_of].transpose(0, 2, 1, 3).reshape(R * s.hv, T, 128)
    vb = vb.reshape(R, T, s.hv, 128).transpose(0, 2, 1, 3).reshape(R * s.hv, T, 128)
    return kb, vb


def check_states(got_t, ref, dtype, what):
    if dtype == torch.float32:
        assert_close_blocks(got_t.float().cpu().numpy(), ref, 2, what)   # per state head
        return
    got = got_t.float().cpu().numpy().astype(np.float64)
    ref = ref.astype(np.float64)
    mag = np.abs(ref)
    ulp = np.exp2(np.floor(np.log2(np.where(mag > 0, mag, 1e-38))) - 7)
    slack = TOL * mag.reshape(mag.shape[0], -1).max(1)[:, None, None]
    assert (np.abs(got - ref) <= ulp + slack).all(), f"{what}: more than one bf16 ulp off"


def test_payload_verify_records_and_outputs(gdn):
    spec = W.shrink(W.ALL_LAYER, layers=2)
    wl = W.make_workload(spec, device="cuda")
    hp = Harness(wl, record_kind=G.RECORD_PAYLOAD)
    hc = Harness(wl)
    pre = wl.state.clone()
    hp.verify_all()
    hc.verify_all()
    torch.cuda.synchronize()
    assert torch.equal(pool_bits(wl.state), pool_bits(pre))
    assert torch.equal(hp.out.view(torch.int32), hc.out.view(torch.int32)), "outputs differ"
    rows = np.arange(spec.rows)
    for layer in range(spec.layers):
        k, v, g, be = payload_fields(hp, layer, rows)
        kin, vin = input_bits(wl, layer, rows)
        assert_bitwise(k, kin, f"layer {layer} payload keys")
        assert_bitwise(v, vin, f"layer {layer} payload values")
        _, _, gc = hc.records(layer, rows)
        assert_bitwise(g, gc, f"layer {layer} payload decays vs correction-record decays")
        gd = OP.gather(wl, layer, rows)
        assert_bitwise(be, gd["beta"], f"layer {layer} payload write strengths")


def _payload_commit(spec, dtype, seed=None):
    kw = {} if seed is None else {"seed": seed}
    wl = W.make_workload(spec, device="cuda", state_dtype=dtype, **kw)
    h = Harness(wl, record_kind=G.RECORD_PAYLOAD)
    pre = wl.state.clone()
    h.verify_all()
    h.commit()
    torch.cuda.synchronize()
    assert h.err_value() == 0
    rows = np.arange(spec.rows)
    live = wl.n_accept > 0
    for layer in range(spec.layers):
        g, res = OP.run_layer(wl, layer, rows, keep=wl.n_accept[:, None], state=pre[layer])
        slots = torch.as_tensor(wl.state_slot[live].astype(np.int64), device="cuda")
        got = wl.state[layer].index_select(0, slots).reshape(-1, 128, 128)
        ref = res.kept[np.repeat(live, spec.hv), 0]
        check_states(got, ref, dtype, f"layer {layer} payload-commit states")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["fp32", "bf16"])
def test_payload_commit(gdn, dtype):
    _payload_commit(W.shrink(W.ALL_LAYER, layers=3), dtype)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["fp32", "bf16"])
def test_payload_commit_longest_windows(gdn, dtype):
    """16 payload records per row (the record capacity's limit), n = 1..16."""
    T = 16
    spec = W.shrink(W.SINGLE_LAYER, rows=8, window=T, rec_tokens=T, n_lo=1, n_hi=T)
    _payload_commit(spec, dtype, seed=96)


def test_payload_commit_align(gdn):
    """Align-mode slots from the oracle's plan (windows that start on, end on
    and cross a block boundary; boundary states written into the source
    slot), payload records, fp32 pool."""
    rng = np.random.default_rng(95)
    rows, blk, max_n = 24, 8, 4
    spec = W.shrink(W.SINGLE_LAYER, rows=rows, hv=4, hk=2, num_slots=256, slot_mode="random")
    wl = W.make_workload(spec, device="cuda", seed=95)
    r = np.tile(np.arange(blk), rows // blk)
    p0 = (8 * rng.integers(3, 9, rows) + r).astype(np.int32)
    n = rng.integers(1, max_n + 1, rows).astype(np.int32)
    n[r >= 5] = 4
    cols = int(((p0 + max_n - 1) // blk).max()) + 1
    table = rng.permutation(spec.num_slots)[: rows * cols].reshape(rows, cols).astype(np.int32)
    src, dst, bl, bs, perr = oracle.align_plan(p0, n, table, blk, max_n)
    assert (perr == 0).all() and ((bs == src) & (bl > 0)).any()
    wl.state_slot = src
    wl.n_accept = n
    h = Harness(wl, record_kind=G.RECORD_PAYLOAD)
    pre = wl.state.clone()
    h.verify_all()
    h.commit(dst=dev_i32(dst), bnd_len=dev_i32(bl), bnd_slot=dev_i32(bs))
    torch.cuda.synchronize()
    assert h.err_value() == 0
    keep = np.stack([n, np.where(bl > 0, bl, -1)], 1)
    g, res = OP.run_layer(wl, 0, np.arange(rows), keep=keep, state=pre[0])
    hv = spec.hv
    fin = wl.state[0].index_select(0, torch.as_tensor(dst.astype(np.int64), device="cuda"))
    check_states(fin.reshape(-1, 128, 128), res.kept[:, 0], torch.float32, "final states")
    has = (bl > 0) & (bs != dst)
    bnd = wl.state[0].index_select(0, torch.as_tensor(bs[has].astype(np.int64), device="cuda"))
    check_states(bnd.reshape(-1, 128, 128), res.kept[np.repeat(has, hv), 1], torch.float32,
                 "boundary states")
