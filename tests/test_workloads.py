"""Host-side checks of the seeded workload generators (no GPU)."""
import numpy as np
import torch

from gated_deltanet_speculative_gdn_amd import workloads as W


def test_deterministic_per_seed():
    a = W.make_workload(W.SINGLE_LAYER)
    b = W.make_workload(W.SINGLE_LAYER)
    assert torch.equal(a.state, b.state) and torch.equal(a.qkv, b.qkv)
    assert np.array_equal(a.n_accept, b.n_accept)
    c = W.make_workload(W.SINGLE_LAYER, seed=7)
    assert not torch.equal(a.state, c.state)


def test_shapes_and_distributions():
    wl = W.make_workload(W.SINGLE_LAYER)
    s = wl.spec
    assert wl.state.shape == (1, 16, 16, 128, 128)
    assert wl.q(0).shape == (64, 8, 128) and wl.v(0).shape == (64, 16, 128)
    assert wl.q(0).stride() == ((2 * 8 + 16) * 128, 128, 1)
    std = wl.state.float().std().item()
    assert 0.048 < std < 0.052
    qn = wl.q(0).float().norm(dim=-1)
    assert torch.allclose(qn, torch.ones_like(qn), atol=1e-2)
    assert (wl.a <= 0).all() and (wl.beta > 0).all() and (wl.beta < 1).all()
    assert wl.n_accept.min() >= s.n_lo and wl.n_accept.max() <= s.n_hi
    assert np.array_equal(wl.state_slot, np.arange(16))


def test_padding_rows_are_null():
    spec = W.shrink(W.MTP_B64, layers=1, num_slots=128)
    wl = W.make_workload(spec)
    pad = np.arange(58, 64)
    assert (wl.state_slot[pad] == -1).all() and (wl.win_len[pad] == 0).all()
    assert (wl.n_accept[pad] == 0).all()
    real = wl.state_slot[:58]
    assert len(set(real.tolist())) == 58 and real.max() < 128


def test_ring_align_offsets_cover_the_special_cases():
    spec = W.shrink(W.RING_ALIGN, layers=1, hv=2, hk=1, dk=8, dv=8)
    wl = W.make_workload(spec)
    r = wl.p0 % 64
    for special in (48, 0, 49, 63):
        assert (r == special).sum() >= 4
    assert wl.block_table.shape[1] >= int((wl.p0.max() + 15) // 64) + 1
    c0 = (wl.p0 - 1) // 64
    rows = np.arange(256)
    assert (wl.block_table[rows, c0] == wl.state_slot).all()
    assert len(set(wl.extra["slots"].reshape(-1).tolist())) == 512


def test_acceptance_rate_counts():
    rng = np.random.default_rng(0)
    n = W.acceptance_rate_counts(rng, 200000, rates=(0.856, 0.694, 0.558))
    assert n.min() >= 1 and n.max() <= 4
    assert abs((n >= 2).mean() - 0.856) < 0.01 and abs((n >= 4).mean() - 0.558) < 0.01


def test_draw_acceptance_rate_counts_on_the_bench_workload():
    """Real rows get n in 1..D from the first D-1 rates; padding rows keep 0; the
    ring workload is refused (its flush commits every record)."""
    wl = W.make_workload(W.WORKLOADS["tiny_l1_b1_h1"])
    W.draw_acceptance_rate_counts(wl)
    assert 1 <= wl.n_accept[0] <= wl.spec.window
    spec = W.MTP_B64
    import dataclasses
    small = dataclasses.replace(spec, layers=1)
    wl = W.make_workload(small)
    W.draw_acceptance_rate_counts(wl)
    real = wl.win_len > 0
    assert (wl.n_accept[~real] == 0).all()
    assert wl.n_accept[real].min() >= 1 and wl.n_accept[real].max() <= spec.window
    again = W.make_workload(small)
    W.draw_acceptance_rate_counts(again)
    assert (again.n_accept == wl.n_accept).all()       # seeded
    ring = dataclasses.replace(W.WORKLOADS["ring_align_l36_b256_l16"], layers=1)
    import pytest
    with pytest.raises(ValueError):
        W.draw_acceptance_rate_counts(W.make_workload(ring))
