"""GPU parity at the interface's limits: the longest windows (T = 8 and 16
records, every position in one window; fp32 and bf16 pools), record
capacities 1, 3, 5 and 13 with align-mode boundaries, a window placed
after pending records (record positions 5..15 verified after positions
0..4), a commit over the most layers a pool set may hold (64), key-head
group sizes 1 to 12, grids that are not a multiple of the XCD count, and a
commit too large for one launch. Bars as in test_parity_gpu."""
import numpy as np
import pytest
import torch

import gated_deltanet_speculative_gdn_amd as G
import oracle
from gated_deltanet_speculative_gdn_amd import workloads as W
from gpu_harness import Harness, dev_i32
from oracle_pool import to_f32
from test_parity_gpu import assert_bitwise, check_layer, pool_bits

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["fp32", "bf16"])
@pytest.mark.parametrize("T", [8, 16])
def test_longest_windows(gdn, T, dtype):
    spec = W.shrink(W.SINGLE_LAYER, rows=8, window=T, rec_tokens=T, n_lo=1, n_hi=T)
    wl = W.make_workload(spec, device="cuda", seed=80 + T, state_dtype=dtype)
    h = Harness(wl)
    pre = wl.state.clone()
    h.verify_all()
    torch.cuda.synchronize()
    assert torch.equal(pool_bits(wl.state), pool_bits(pre))
    h.commit()
    torch.cuda.synchronize()
    assert h.err_value() == 0
    check_layer(h, 0, np.arange(spec.rows), wl.n_accept, pre[0])


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["fp32", "bf16"])
@pytest.mark.parametrize("T", [1, 3, 5, 13])
def test_odd_record_capacities_with_boundaries(gdn, T, dtype):
    """Record capacities off the 4/8/16 grid (the smaller members of each
    compiled window capacity, so the commit's record staging meets partial
    chunks), windows of T tokens, n from 1 to T (first row n = T, second
    n = 1), and an align-mode boundary state after n - 1 tokens, written to a
    spare slot, for every row with n >= 2."""
    rows = 12
    spec = W.shrink(W.SINGLE_LAYER, rows=rows, window=T, rec_tokens=T, n_lo=1, n_hi=T,
                    num_slots=2 * rows)
    wl = W.make_workload(spec, device="cuda", seed=120 + T, state_dtype=dtype)
    n = wl.n_accept.copy()
    n[0], n[1] = T, 1
    h = Harness(wl)
    pre = wl.state.clone()
    h.verify_all()
    torch.cuda.synchronize()
    assert torch.equal(pool_bits(wl.state), pool_bits(pre))
    bl = np.where(n >= 2, n - 1, 0).astype(np.int32)
    spare = np.setdiff1d(np.arange(spec.num_slots), wl.state_slot)[:rows]
    assert len(spare) == rows
    bs = np.where(bl > 0, spare, -1).astype(np.int32)
    h.commit(n=dev_i32(n), bnd_len=dev_i32(bl), bnd_slot=dev_i32(bs))
    torch.cuda.synchronize()
    assert h.err_value() == 0
    check_layer(h, 0, np.arange(rows), n, pre[0], bnd=(bl, bs))


def test_window_after_pending_records(gdn):
    """Positions 0..4 verified first, then positions 5..15 with the first five
    records pending (ring base 5, window 11, T = 16): together the outputs and
    records of one 16-token window, checked against the native rule over all
    16 tokens, then a commit of n = 1..16."""
    T = 16
    spec = W.shrink(W.SINGLE_LAYER, rows=8, window=T, rec_tokens=T, n_lo=1, n_hi=T)
    wl = W.make_workload(spec, device="cuda", seed=90)
    h = Harness(wl)
    pre = wl.state.clone()
    rows = spec.rows
    first = dev_i32(np.full(rows, 5))
    second = dev_i32(np.full(rows, T - 5))
    base0 = dev_i32(np.zeros(rows))
    base5 = dev_i32(np.full(rows, 5))
    ts0 = dev_i32(wl.tok_start)
    ts5 = dev_i32(wl.tok_start + 5)
    for ts, w, base in ((ts0, first, base0), (ts5, second, base5)):
        G.gdn_verify(h.pools, 0, h.state_slot, h.rec_slot, ts, w, base, wl.q(0), wl.k(0),
                     wl.v(0), wl.a[0], wl.beta[0], h.out[0], err_flags=h.err)
    torch.cuda.synchronize()
    assert torch.equal(pool_bits(wl.state), pool_bits(pre))
    h.commit()
    torch.cuda.synchronize()
    assert h.err_value() == 0
    check_layer(h, 0, np.arange(rows), wl.n_accept, pre[0])


def test_commit_over_64_layers(gdn):
    spec = W.shrink(W.ALL_LAYER, layers=G.GDN_MAX_LAYERS, rows=3, hv=2, hk=1, num_slots=8)
    wl = W.make_workload(spec, device="cuda", seed=91)
    h = Harness(wl)
    pre = wl.state.clone()
    h.verify_all()
    h.commit()
    torch.cuda.synchronize()
    assert h.err_value() == 0
    for layer in range(spec.layers):
        check_layer(h, layer, np.arange(spec.rows), wl.n_accept, pre[layer])


@pytest.mark.parametrize("hv,hk", [(8, 2), (6, 6), (6, 3), (12, 1)],
                         ids=["group4", "group1", "hv6_group2", "group12"])
def test_key_head_groups(gdn, hv, hk):
    """Value head h reads key head h / (HV/HK) for group sizes 1, 2, 4 and 12,
    including a head count that is not a power of two; 7 rows on random slots."""
    spec = W.shrink(W.SINGLE_LAYER, rows=7, hv=hv, hk=hk, num_slots=32, slot_mode="random")
    wl = W.make_workload(spec, device="cuda", seed=100 + hv * 16 + hk)
    h = Harness(wl)
    pre = wl.state.clone()
    h.verify_all()
    h.commit()
    torch.cuda.synchronize()
    assert h.err_value() == 0
    check_layer(h, 0, np.arange(spec.rows), wl.n_accept, pre[0])


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["fp32", "bf16"])
def test_grids_not_a_multiple_of_the_xcd_count(gdn, dtype):
    """Launches whose workgroup count is not a multiple of the 8 XCDs, so the
    XCD-contiguous id remap leaves a tail of ids mapped to themselves: 3 layers
    x 5 rows x 3 value heads gives verify grids of 30 (tail 6) and, on bf16
    pools (4 workgroups per head), a commit grid of 180 (tail 4). Every layer
    against the oracle, every slot outside the write set unchanged."""
    spec = W.shrink(W.ALL_LAYER, layers=3, rows=5, hv=3, hk=3, num_slots=16)
    wl = W.make_workload(spec, device="cuda", state_dtype=dtype, seed=131)
    h = Harness(wl)
    pre = wl.state.clone()
    h.verify_all()
    h.commit()
    torch.cuda.synchronize()
    assert h.err_value() == 0
    for layer in range(spec.layers):
        check_layer(h, layer, np.arange(spec.rows), wl.n_accept, pre[layer])
    live = {int(s) for s, n in zip(wl.state_slot, wl.n_accept) if n > 0}
    for layer in range(spec.layers):
        for s in range(spec.num_slots):
            if s not in live:
                assert torch.equal(pool_bits(wl.state[layer, s]), pool_bits(pre[layer, s])), (layer, s)


@pytest.mark.parametrize("dtype,rows", [(torch.float32, 21846), (torch.bfloat16, 43691)],
                         ids=["fp32", "bf16"])
def test_commit_beyond_one_launch(gdn, dtype, rows):
    """An all-layer commit whose grid passes the 2^32 - 1 work-items one launch
    may hold: 3 layers x rows x 32 value heads is 16,777,728 workgroups on fp32
    pools (8 per head) and 16,777,344 on bf16 pools (4 per head), so the
    library issues two launches, layers 0-1 and layer 2. Five live rows per
    layer, at the start, the middle and the end (the last is the grid's last
    workgroup), in place and into other slots; every other row n = 0. The
    records are seeded directly (corrections, unit keys, decays in (0.2, 1)):
    every committed head equals the oracle's replay of them bit for bit (bf16
    pools: its RNE), and every other slot is unchanged."""
    L, HV, HK, T = 3, 32, 16, 4
    live = np.array([0, 1, rows // 2, rows - 2, rows - 1])
    nl = len(live)
    num_slots = 2 * nl
    print(f"commit over {L * rows * HV} heads, {dtype}", flush=True)
    gen = torch.Generator(device="cuda").manual_seed(140)
    state = (torch.randn((L, num_slots, HV, 128, 128), generator=gen, device="cuda")
             * 0.05).to(dtype)
    d = torch.randn((L, nl, HV, T, 128), generator=gen, device="cuda") * 0.1
    k = torch.nn.functional.normalize(
        torch.randn((L, nl, HV, T, 128), generator=gen, device="cuda"), dim=-1)
    g = torch.rand((L, nl, HV, T), generator=gen, device="cuda") * 0.8 + 0.2
    rec = G.Pools.alloc_records(L, nl, HV, T)
    rec[..., : T * 128] = d.reshape(L, nl, HV, T * 128)
    rec[..., T * 128: 2 * T * 128] = k.reshape(L, nl, HV, T * 128)
    rec[..., 2 * T * 128: 2 * T * 128 + T] = g
    pools = G.Pools(state, rec, HK, T)
    src = np.full(rows, -1, np.int32)
    dst = np.full(rows, -1, np.int32)
    rs = np.zeros(rows, np.int32)
    n = np.zeros(rows, np.int32)
    src[live] = np.arange(nl)
    dst[live] = [0, nl + 1, 2, nl + 3, nl + 4]          # in place and moved
    rs[live] = np.arange(nl)
    n[live] = [4, 1, 3, 2, 4]
    pre = state.clone()
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    G.gdn_commit_all_layers(pools, dev_i32(src), dev_i32(dst), dev_i32(rs), dev_i32(n),
                            err_flags=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    written = set(int(x) for x in dst[live])
    for layer in range(L):
        for i, b in enumerate(live):
            S0 = to_f32(pre[layer, src[b]]).reshape(HV, 128, 128)
            rep = oracle.replay_heads(S0, np.full(HV, n[b], np.int32),
                                      d[layer, i].cpu().numpy(), k[layer, i].cpu().numpy(),
                                      g[layer, i].cpu().numpy())
            got = state[layer, dst[b]]
            if dtype == torch.float32:
                assert_bitwise(got.cpu().numpy().reshape(HV, 128, 128), rep,
                               f"layer {layer} row {b}")
            else:
                bits_ = got.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
                assert_bitwise(bits_.reshape(HV, 128, 128), oracle.f32_to_bf16_rne(rep),
                               f"layer {layer} row {b}")
        keep = [s for s in range(num_slots) if s not in written]
        idx = torch.as_tensor(keep, device="cuda")
        assert torch.equal(pool_bits(state[layer].index_select(0, idx)),
                           pool_bits(pre[layer].index_select(0, idx))), f"layer {layer}"


def test_bf16_commit_rounding_across_the_fp32_range(gdn):
    """The bf16 commit rounds each final state value once, to nearest even
    (vLLM RecoverSSM PR, Test Plan: bf16 state). Records seeded directly: a
    zero checkpoint, decay 1, corrections with random full 24-bit mantissas,
    and keys that are signed powers of two from 2^-134 to 2^120, so the
    committed value fma(delta[v], key[k], 0) is delta[v] scaled exactly (or
    rounded once into the fp32 subnormal range) across the whole fp32 range:
    fp32 subnormals, bf16 ties of both parities, values that round up into the
    next binade or overflow to infinity, infinite corrections. Every stored bf16
    value equals the oracle's integer RNE of the oracle's replay bit for bit
    (NaN corrections: a NaN, whose payload IEEE leaves open)."""
    rng = np.random.default_rng(151)
    rows, HV, T = 4, 8, 1
    H = rows * HV
    m = rng.integers(0, 1 << 23, size=(H, 128), dtype=np.uint32)
    e = rng.integers(127 - 12, 127 + 12, size=(H, 128), dtype=np.uint32)
    s = rng.integers(0, 2, size=(H, 128), dtype=np.uint32)
    m[:, :16] = (m[:, :16] & ~np.uint32(0xffff)) | np.uint32(0x8000)        # exact ties
    m[:, 16:24] = (m[:, 16:24] & ~np.uint32(0xffff)) | np.uint32(0x7fff)    # just below
    m[:, 24:32] = (m[:, 24:32] & ~np.uint32(0xffff)) | np.uint32(0x8001)    # just above
    m[:, 32:36] = np.uint32(0x7fffff)                                       # round to next binade
    delta = ((s << 31) | (e << 23) | m).view(np.float32).copy()
    delta[0, 40] = np.inf
    delta[1, 41] = -np.inf
    delta[2, 42] = np.nan
    kexp = -134 + 2 * np.arange(128)                                       # 2^-134 .. 2^120
    keys = np.ldexp(np.where(np.arange(128) % 3 == 0, -1.0, 1.0), kexp).astype(np.float32)
    keys = np.broadcast_to(keys, (H, 128)).copy()
    state = torch.zeros((1, rows, HV, 128, 128), dtype=torch.bfloat16, device="cuda")
    rec = G.Pools.alloc_records(1, rows, HV, T)
    rec[0, :, :, :128] = torch.as_tensor(delta.reshape(rows, HV, 128), device="cuda")
    rec[0, :, :, 128:256] = torch.as_tensor(keys.reshape(rows, HV, 128), device="cuda")
    rec[0, :, :, 256] = 1.0
    pools = G.Pools(state, rec, HV, T)
    slots = dev_i32(np.arange(rows))
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    G.gdn_commit_all_layers(pools, slots, slots, slots, dev_i32(np.ones(rows)), err_flags=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    want = oracle.replay_heads(np.zeros((H, 128, 128), np.float32), np.ones(H, np.int32),
                               delta[:, None, :], keys[:, None, :], np.ones((H, 1), np.float32))
    assert np.isinf(want).any() and (np.abs(want[np.isfinite(want)]) < 2.0 ** -126).any()
    want_bits = oracle.f32_to_bf16_rne(want)
    got_bits = state.view(torch.int16).cpu().numpy().view(np.uint16).reshape(H, 128, 128)
    nan = np.isnan(want)
    assert np.array_equal(got_bits[~nan], want_bits[~nan]), int((got_bits != want_bits)[~nan].sum())
    got_nan = ((got_bits & 0x7f80) == 0x7f80) & ((got_bits & 0x7f) != 0)
    assert got_nan[nan].all()
