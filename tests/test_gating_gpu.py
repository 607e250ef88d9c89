"""GPU parity of verify's upstream-fusion options: gates formed in the kernel
from the raw gate projections a, b with per-head A_log and dt_bias, and the
output rounded to bf16 and written into a strided view of a wider layer output
(vLLM RecoverSSM PR, Commits item 2: the verify reads strided views of the
conv output and writes straight into the layer output).

Bars: as the other parity tests (normwise relative error <= 1e-5 per layer
against the oracle's native per-token rule, fed with the oracle's own gates
from the same raw inputs; the commit bit-exact against the oracle's replay of
the GPU records). bf16 outputs: bit-identical to the round-to-nearest-even of
the same kernel's fp32 outputs, and within one bf16 ulp (+ the fp32
tolerance) of the oracle's fp32 outputs.
"""
import copy

import numpy as np
import pytest
import torch

import oracle
import oracle_pool as OP
import gated_deltanet_speculative_gdn_amd as G
from gated_deltanet_speculative_gdn_amd import workloads as W
from gpu_harness import Harness
from test_parity_gpu import TOL, assert_bitwise, check_layer, pool_bits

pytestmark = pytest.mark.gpu


def oracle_gated(wl, rg):
    """A view of the workload whose a / beta are the oracle's log-gates and
    write strengths from the raw inputs (state and q/k/v shared)."""
    lg = np.empty(tuple(rg.a.shape), np.float32)
    be = np.empty_like(lg)
    for layer in range(wl.spec.layers):
        lg[layer], be[layer] = oracle.raw_gates(rg.a[layer].cpu().numpy(), rg.b[layer].cpu().numpy(),
                                                rg.A_log[layer].cpu().numpy(),
                                                rg.dt_bias[layer].cpu().numpy())
    w2 = copy.copy(wl)
    w2.a = torch.as_tensor(lg, device=wl.a.device)
    w2.beta = torch.as_tensor(be, device=wl.a.device)
    return w2


def verify_raw(h, rg, layer, out=None):
    wl = h.wl
    G.gdn_verify(h.pools, layer, h.state_slot, h.rec_slot, h.tok_start, h.win_len, None,
                 wl.q(layer), wl.k(layer), wl.v(layer), rg.a[layer], rg.b[layer],
                 h.out[layer] if out is None else out, A_log=rg.A_log[layer],
                 dt_bias=rg.dt_bias[layer], err_flags=h.err)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["fp32", "bf16"])
def test_raw_gates_match_oracle(gdn, dtype):
    spec = W.shrink(W.ALL_LAYER, layers=3)
    wl = W.make_workload(spec, device="cuda", state_dtype=dtype)
    rg = W.make_raw_gates(wl, device="cuda")
    h = Harness(wl)
    pre = wl.state.clone()
    for layer in range(spec.layers):
        verify_raw(h, rg, layer)
    torch.cuda.synchronize()
    assert torch.equal(pool_bits(wl.state), pool_bits(pre)), "verify wrote the checkpoint"
    h.commit()
    torch.cuda.synchronize()
    assert h.err_value() == 0
    h.wl = oracle_gated(wl, rg)
    rows = np.arange(spec.rows)
    for layer in range(spec.layers):
        check_layer(h, layer, rows, wl.n_accept, pre[layer])


def test_raw_gates_extreme_inputs(gdn):
    """Raw inputs on both softplus branches (a + dt_bias far above 20 gives a
    decay of 0; far below gives a decay of 1 to fp32) and saturated write
    strengths."""
    spec = W.shrink(W.SINGLE_LAYER, layers=1)
    wl = W.make_workload(spec, device="cuda", seed=61)
    rg = W.make_raw_gates(wl, device="cuda", seed=61)
    a = rg.a[0]
    a[0::4] = 40.0
    a[1::4] = -60.0
    rg.b[0][2::4] = 30.0
    rg.b[0][3::4] = -30.0
    h = Harness(wl)
    pre = wl.state.clone()
    verify_raw(h, rg, 0)
    h.commit()
    torch.cuda.synchronize()
    assert h.err_value() == 0
    h.wl = oracle_gated(wl, rg)
    check_layer(h, 0, np.arange(spec.rows), wl.n_accept, pre[0])


def test_bf16_output_into_layer_view(gdn):
    spec = W.shrink(W.SINGLE_LAYER, layers=1)
    wl = W.make_workload(spec, device="cuda", seed=62)
    rg = W.make_raw_gates(wl, device="cuda", seed=62)
    T, HV = wl.tokens, spec.hv
    h = Harness(wl)
    verify_raw(h, rg, 0)                      # fp32 outputs into h.out[0]
    # a wider bf16 layer output [tokens][HV*128 + 64]; the heads sit at column 32
    big = torch.full((T, HV * 128 + 64), float("nan"), dtype=torch.bfloat16, device="cuda")
    view = big[:, 32: 32 + HV * 128].view(T, HV, 128)
    verify_raw(h, rg, 0, out=view)
    torch.cuda.synchronize()
    assert h.err_value() == 0
    f32 = h.out[0].cpu().numpy()
    got = view.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    assert_bitwise(got, oracle.f32_to_bf16_rne(f32), "bf16 outputs vs RNE of the fp32 outputs")
    assert torch.isnan(big[:, :32]).all() and torch.isnan(big[:, 32 + HV * 128:]).all()
    # against the oracle's fp32 outputs: one bf16 ulp plus the fp32 tolerance
    rows = np.arange(spec.rows)
    g, res = OP.run_layer(oracle_gated(wl, rg), 0, rows)
    tok = OP.token_index(wl, rows)
    o = oracle.bf16_to_f32(got)[tok.reshape(-1)].reshape(len(rows), tok.shape[1], HV, 128)
    o = o.transpose(0, 2, 1, 3).reshape(len(rows) * HV, tok.shape[1], 128).astype(np.float64)
    ref = res.o.astype(np.float64)
    mag = np.abs(ref)
    ulp = np.exp2(np.floor(np.log2(np.where(mag > 0, mag, 1e-38))) - 7)
    slack = TOL * np.abs(ref).max()
    assert (np.abs(o - ref) <= ulp + slack).all(), "bf16 outputs: more than one ulp off"


def test_raw_gates_with_payload_records(gdn):
    """Raw-input gating and payload records together: the payload keeps the
    decay and write strength formed in the kernel (bit-identical to the
    correction record's decay from the same raw inputs), and the payload commit
    lands within the fp32 tolerance of the oracle fed with its own gates."""
    from test_payload_gpu import check_states, payload_fields
    spec = W.shrink(W.ALL_LAYER, layers=2)
    wl = W.make_workload(spec, device="cuda")
    rg = W.make_raw_gates(wl, device="cuda")
    hp = Harness(wl, record_kind=G.RECORD_PAYLOAD)
    hc = Harness(wl)
    pre = wl.state.clone()
    for layer in range(spec.layers):
        verify_raw(hp, rg, layer)
        verify_raw(hc, rg, layer)
    torch.cuda.synchronize()
    assert torch.equal(hp.out.view(torch.int32), hc.out.view(torch.int32)), "outputs differ"
    rows = np.arange(spec.rows)
    og = oracle_gated(wl, rg)
    for layer in range(spec.layers):
        _, _, g, be = payload_fields(hp, layer, rows)
        _, _, gc = hc.records(layer, rows)
        assert_bitwise(g, gc, f"layer {layer} payload decays vs correction-record decays")
        gd = OP.gather(og, layer, rows)
        np.testing.assert_allclose(be, gd["beta"], rtol=1e-6, atol=0,
                                   err_msg=f"layer {layer} payload write strengths")
    hp.commit()
    torch.cuda.synchronize()
    assert hp.err_value() == 0
    live = wl.n_accept > 0
    for layer in range(spec.layers):
        _, res = OP.run_layer(og, layer, rows, keep=wl.n_accept[:, None], state=pre[layer])
        slots = torch.as_tensor(wl.state_slot[live].astype(np.int64), device="cuda")
        got = wl.state[layer].index_select(0, slots).reshape(-1, 128, 128)
        check_states(got, res.kept[np.repeat(live, spec.hv), 0], torch.float32,
                     f"layer {layer} payload-commit states with raw gates")
