"""The variants at the bench's launch configuration: 48 layers, batch 64 with
6 graph-padding rows, 32/16 heads, 4-token windows, fp32 state (the workload
`bench.py --gating channel`, `--record payload` and `--conv` time). Every layer is verified and one commit launch covers all 48 layers;
layers 0, 23 and 47 are checked against the oracle (sampled outputs, as the
oracle computes them head by head), with the bars of test_channel_gpu and
test_payload_gpu; padding rows write nothing."""
import numpy as np
import pytest
import torch

import oracle_pool as OP
import gated_deltanet_speculative_gdn_amd as G
from gated_deltanet_speculative_gdn_amd import workloads as W
from gpu_harness import Harness
from test_channel_gpu import check_channel_layer, verify_ch
from test_parity_gpu import pool_bits
from test_payload_gpu import check_states

pytestmark = pytest.mark.gpu

LAYERS = (0, 23, 47)


def split_rows(wl):
    real = np.nonzero(wl.state_slot >= 0)[0]
    pad = np.nonzero(wl.state_slot < 0)[0]
    assert len(real) == 58 and len(pad) == 6
    return real, pad


def padding_untouched(h, wl, pad):
    tok = (wl.tok_start[pad][:, None] + np.arange(wl.spec.window)[None]).reshape(-1)
    assert torch.isnan(h.out[:, torch.as_tensor(tok, device="cuda")]).all(), "padding outputs"


def test_channel_decays_at_bench_size(gdn):
    spec = W.MTP_B64
    wl = W.make_workload(spec, device="cuda")
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
    real, pad = split_rows(wl)
    for layer in LAYERS:
        check_channel_layer(h, a_ch, layer, real, wl.n_accept[real], pre[layer])
    padding_untouched(h, wl, pad)


def test_payload_records_at_bench_size(gdn):
    spec = W.MTP_B64
    wl = W.make_workload(spec, device="cuda")
    h = Harness(wl, record_kind=G.RECORD_PAYLOAD)
    pre = wl.state.clone()
    h.verify_all()
    torch.cuda.synchronize()
    assert torch.equal(pool_bits(wl.state), pool_bits(pre)), "verify wrote the checkpoint"
    h.commit()
    torch.cuda.synchronize()
    assert h.err_value() == 0
    real, pad = split_rows(wl)
    n = wl.n_accept[real]
    live = n > 0
    slots = torch.as_tensor(wl.state_slot[real][live].astype(np.int64), device="cuda")
    for layer in LAYERS:
        _, res = OP.run_layer(wl, layer, real, keep=n[:, None], state=pre[layer])
        got = wl.state[layer].index_select(0, slots).reshape(-1, 128, 128)
        check_states(got, res.kept[np.repeat(live, spec.hv), 0], torch.float32,
                     f"layer {layer} payload-commit states")
        # rows that accepted nothing keep their checkpoint bit for bit
        idle = torch.as_tensor(wl.state_slot[real][~live].astype(np.int64), device="cuda")
        if idle.numel():
            assert torch.equal(pool_bits(wl.state[layer].index_select(0, idle)),
                               pool_bits(pre[layer].index_select(0, idle)))
    padding_untouched(h, wl, pad)


def test_conv_compaction_at_bench_size(gdn):
    """The short-conv compaction in the same launch as the all-layer commit, at
    the bench's configuration (`bench.py --conv`): the state-replay part equals
    a plain commit of a copy of the pools bit for bit, and every layer's conv
    pool equals the oracle's token walk bit for bit (padding rows move
    nothing)."""
    from test_conv_commit_gpu import expected_pool, raw
    spec = W.MTP_B64
    wl = W.make_workload(spec, device="cuda")
    cv = W.make_conv(wl, state_len=3, dtype=torch.bfloat16, device="cuda")
    h = Harness(wl)
    h.verify_all()
    torch.cuda.synchronize()
    ref_state = wl.state.clone()
    ref_pools = G.Pools(ref_state, h.rec, spec.hk, spec.rec_tokens)
    G.gdn_commit_all_layers(ref_pools, h.state_slot, h.state_slot, h.rec_slot, h.n_accept,
                            err_flags=h.err)
    pre = raw(cv.state)
    x = raw(cv.x)
    G.gdn_commit_all_layers_conv(h.pools, G.ConvPools(cv.state, cv.x), h.state_slot, h.state_slot,
                                 h.rec_slot, h.n_accept, conv_tok_start=h.tok_start, err_flags=h.err)
    torch.cuda.synchronize()
    assert h.err_value() == 0
    assert torch.equal(pool_bits(wl.state), pool_bits(ref_state)), "state replay differs"
    got = raw(cv.state)
    for layer in range(spec.layers):
        exp = expected_pool(pre[layer], x[layer], range(spec.rows), wl.state_slot, wl.state_slot,
                            wl.n_accept, wl.tok_start)
        np.testing.assert_array_equal(got[layer], exp, err_msg=f"layer {layer}")
