"""The entry points are stream-ordered and capturable in a HIP graph (the
verify launches run inside a captured decode graph: vLLM RecoverSSM PR,
Purpose). Verify of every layer, the all-layer commit into distinct
destination slots and the align plan are captured once and replayed three
times, with eager work (clearing the outputs) and synchronisations between
the replays; every replay must equal the eager result bit for bit."""
import numpy as np
import pytest
import torch

import gated_deltanet_speculative_gdn_amd as G
from gated_deltanet_speculative_gdn_amd import workloads as W
from gpu_harness import Harness, dev_i32
from test_parity_gpu import pool_bits

pytestmark = pytest.mark.gpu
NAN = float("nan")


def test_verify_commit_and_plan_replayed_from_a_graph(gdn):
    spec = W.shrink(W.ALL_LAYER, layers=3, rows=8, num_slots=32)
    wl = W.make_workload(spec, device="cuda", seed=77)
    h = Harness(wl)
    used = set(int(x) for x in wl.state_slot)
    free = [x for x in range(spec.num_slots) if x not in used][: spec.rows]
    dst = dev_i32(np.asarray(free))
    rng = np.random.default_rng(77)
    p0 = dev_i32(rng.integers(1, 500, spec.rows))
    n = dev_i32(rng.integers(0, 5, spec.rows))
    table = dev_i32(rng.permutation(4096)[: spec.rows * 16].reshape(spec.rows, 16))
    plan_out = [torch.empty(spec.rows, dtype=torch.int32, device="cuda") for _ in range(4)]

    def work():
        h.verify_all()
        h.commit(dst=dst)
        G.gdn_align_plan(p0, n, table, 64, 4, *plan_out, err_flags=h.err)

    def clear():
        h.out.fill_(NAN)
        h.rec.fill_(NAN)
        for t in plan_out:
            t.fill_(-7)
        for layer in range(spec.layers):
            wl.state[layer].index_fill_(0, dst.long(), NAN)

    clear()
    work()
    torch.cuda.synchronize()
    assert h.err_value() == 0
    ref = (h.out.clone(), h.rec.clone(), pool_bits(wl.state).clone(), [t.clone() for t in plan_out])

    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        clear()
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=side):
            work()
    torch.cuda.synchronize()
    for replay in range(3):
        clear()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(h.out.view(torch.int32), ref[0].view(torch.int32)), f"replay {replay}: outputs"
        assert torch.equal(h.rec.view(torch.int32), ref[1].view(torch.int32)), f"replay {replay}: records"
        assert torch.equal(pool_bits(wl.state), ref[2]), f"replay {replay}: committed states"
        for a, b in zip(plan_out, ref[3]):
            assert torch.equal(a, b), f"replay {replay}: align plan"
    assert h.err_value() == 0
