"""The library keeps no state between calls: verify of different layers issued
concurrently from two host threads on two HIP streams gives, bit for bit, the
outputs and records of the same calls issued one after another on one stream;
the all-layer commit that follows agrees as well."""
import threading

import numpy as np
import pytest
import torch

import gated_deltanet_speculative_gdn_amd as G
from gated_deltanet_speculative_gdn_amd import workloads as W
from gpu_harness import Harness
from test_parity_gpu import pool_bits

pytestmark = pytest.mark.gpu


def test_two_threads_two_streams_match_serial(gdn):
    spec = W.shrink(W.ALL_LAYER, layers=6)
    wl = W.make_workload(spec, device="cuda", seed=55)
    pre = wl.state.clone()
    serial = Harness(wl)
    serial.verify_all()
    serial.commit()
    torch.cuda.synchronize()
    ref = (serial.out.clone(), serial.rec.clone(), pool_bits(wl.state).clone())

    wl.state.copy_(pre)
    conc = Harness(wl)
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    errors = []

    def work(i):
        try:
            with torch.cuda.stream(streams[i]):
                for layer in range(i, spec.layers, 2):
                    conc.verify_layer(layer)
            streams[i].synchronize()
        except Exception as e:           # reported by the main thread
            errors.append(e)

    torch.cuda.synchronize()
    threads = [threading.Thread(target=work, args=(i,)) for i in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors
    conc.commit()
    torch.cuda.synchronize()
    assert conc.err_value() == 0
    assert torch.equal(conc.out.view(torch.int32), ref[0].view(torch.int32)), "outputs differ"
    assert torch.equal(conc.rec.view(torch.int32), ref[1].view(torch.int32)), "records differ"
    assert torch.equal(pool_bits(wl.state), ref[2]), "committed states differ"
