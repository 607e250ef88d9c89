"""Pins for the CPU oracle (no GPU).

Each test checks the oracle against something other than itself: the four
invariants of the method, closed forms of the gated delta rule, the
transition-matrix form of the rule evaluated in fp64, one-hot inputs whose
reductions have a single term, the page's record-size figure, hand-worked
align plans, an independent closed form of the align plan, and torch's bf16
rounding. The per-key-channel decay variant (the KDA reading) is pinned to the
scalar rule (a decay repeated over the channels gives it bit for bit), to its
own replay, to the per-column closed form at beta = 0 and to its fp64
transition-matrix form. A dropped term, a wrong sign, a transposed operand or a wrong index
in the oracle fails at least one of them.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle

F32 = np.float32
HERE = os.path.dirname(os.path.abspath(__file__))


def _inputs(seed, H=3, T=4, K=16, V=12, extreme=False):
    rng = np.random.default_rng(seed)
    S0 = rng.normal(0, 0.05, (H, V, K)).astype(F32)
    q = rng.normal(size=(H, T, K)).astype(F32)
    k = rng.normal(size=(H, T, K)).astype(F32)
    v = rng.normal(size=(H, T, V)).astype(F32)
    a = (-np.logaddexp(0, rng.normal(size=(H, T)))).astype(F32)
    beta = (1 / (1 + np.exp(-rng.normal(size=(H, T))))).astype(F32)
    if extreme:
        a[:, 0] = 0.0            # no decay
        a[:, 1] = -100.0         # decay to the subnormal range
        beta[:, 2] = 1.0
        beta[:, 3] = 0.0
    return S0, q, k, v, a, beta


def _norm64(x, eps=oracle.EPS):
    x = np.asarray(x, np.float64)
    return x / np.sqrt((x * x).sum(-1, keepdims=True) + np.float64(F32(eps)))


def _relerr(x, y):
    x, y = np.asarray(x, np.float64), np.asarray(y, np.float64)
    return float(np.abs(x - y).max() / max(np.abs(y).max(), 1e-300))


# --------------------------------------------------------------------------
# The four invariants of the method
# --------------------------------------------------------------------------

@pytest.mark.parametrize("seed", [0, 1, 2])
@pytest.mark.parametrize("K,V,T", [(4, 4, 4), (16, 12, 5), (128, 128, 4)])
def test_replay_of_accepted_prefix_equals_native_state(seed, K, V, T):
    """Replaying the first n records onto the checkpoint gives S_n of the native
    rule, bit for bit, for every n = 0..w."""
    S0, q, k, v, a, beta = _inputs(seed, H=2, T=T, K=K, V=V)
    w = np.array([T, T - 1], np.int32)
    r = oracle.native_heads(S0, w, q, k, v, a, beta, snaps=True)
    for h in range(2):
        for n in range(w[h] + 1):
            got = oracle.replay_heads(S0[h:h + 1], [n], r.rec_delta[h:h + 1],
                                      r.rec_khat[h:h + 1], r.rec_g[h:h + 1])[0]
            want = S0[h] if n == 0 else r.snaps[h, n - 1]
            assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), (h, n)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_zero_accepted_leaves_state_bit_identical(seed):
    S0, q, k, v, a, beta = _inputs(seed)
    r = oracle.native_heads(S0, np.full(3, 4, np.int32), q, k, v, a, beta,
                            keep=np.zeros((3, 1), np.int32))
    got = oracle.replay_heads(S0, np.zeros(3, np.int32), r.rec_delta, r.rec_khat, r.rec_g)
    assert np.array_equal(got.view(np.uint32), S0.view(np.uint32))
    assert np.array_equal(r.kept[:, 0].view(np.uint32), S0.view(np.uint32))


def test_verify_never_modifies_checkpoint():
    S0, q, k, v, a, beta = _inputs(3)
    before = S0.copy()
    oracle.native_heads(S0, np.full(3, 4, np.int32), q, k, v, a, beta, snaps=True)
    assert np.array_equal(S0.view(np.uint32), before.view(np.uint32))


def test_zero_length_window_writes_nothing():
    """A padding head (w = 0) produces no output, no record and no state."""
    S0, q, k, v, a, beta = _inputs(4)
    w = np.array([4, 0, 2], np.int32)
    r = oracle.native_heads(S0, w, q, k, v, a, beta, snaps=True,
                            keep=np.array([[4], [0], [2]], np.int32))
    assert not r.o[1].any() and not r.rec_delta[1].any() and not r.rec_khat[1].any()
    assert not r.rec_g[1].any() and not r.snaps[1].any()
    assert np.array_equal(r.kept[1, 0], S0[1])
    assert not r.o[2, 2:].any() and not r.snaps[2, 2:].any()


# --------------------------------------------------------------------------
# Closed forms of the gated delta rule
# --------------------------------------------------------------------------

def test_no_write_no_decay_keeps_state_and_reads_it():
    """beta = 0, g = 1: the state never changes; o_t = S0 q_hat_t."""
    S0, q, k, v, a, beta = _inputs(5)
    a[:] = 0
    beta[:] = 0
    r = oracle.native_heads(S0, np.full(3, 4, np.int32), q, k, v, a, beta, snaps=True)
    for t in range(4):
        assert np.array_equal(r.snaps[:, t], S0)
    want = np.einsum("hvk,htk->htv", S0.astype(np.float64), _norm64(q))
    assert _relerr(r.o, want) < 1e-6


def test_no_write_is_pure_decay():
    """beta = 0: S_n = (((S0 g_1) g_2) ...), each product rounded once."""
    S0, q, k, v, a, beta = _inputs(6)
    beta[:] = 0
    r = oracle.native_heads(S0, np.full(3, 4, np.int32), q, k, v, a, beta, snaps=True)
    h = S0.copy()
    for t in range(4):
        h = (h * r.rec_g[:, t][:, None, None]).astype(F32)
        assert np.array_equal(r.snaps[:, t], h)
        assert not r.rec_delta[:, t].any()


def test_full_forget_writes_rank_one():
    """g = 0 (a = -inf): u = 0, delta = beta v, S_1 = delta k_hat^T exactly."""
    S0, q, k, v, a, beta = _inputs(7)
    a[:, 0] = -np.inf
    r = oracle.native_heads(S0, np.full(3, 1, np.int32), q, k, v, a, beta, snaps=True)
    assert np.all(r.rec_g[:, 0] == 0)
    delta = (beta[:, 0][:, None] * v[:, 0]).astype(F32)
    assert np.array_equal(r.rec_delta[:, 0], delta)
    want = (delta[:, :, None] * r.rec_khat[:, 0][:, None, :]).astype(F32)
    assert np.array_equal(r.snaps[:, 0], want)


def test_delta_rule_with_unit_strength_stores_the_value():
    """beta = 1, g = 1, q = k: the update writes v at key k_hat, so o = v
    (up to the normalisation epsilon and fp32 rounding)."""
    S0, q, k, v, a, beta = _inputs(8, K=128, V=128)
    a[:] = 0
    beta[:] = 1
    r = oracle.native_heads(S0, np.full(3, 1, np.int32), k, k, v, a, beta)
    assert _relerr(r.o[:, 0], v[:, 0]) < 1e-5


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_one_step_identity(seed):
    """S_1 k_hat = g (1 - beta |k_hat|^2) S0 k_hat + beta |k_hat|^2 v."""
    S0, q, k, v, a, beta = _inputs(seed, K=128, V=128)
    r = oracle.native_heads(S0, np.full(3, 1, np.int32), q, k, v, a, beta, snaps=True)
    kh = _norm64(k[:, 0])
    n2 = (kh * kh).sum(-1)
    g = np.exp(a[:, 0].astype(np.float64))
    b = beta[:, 0].astype(np.float64)
    lhs = np.einsum("hvk,hk->hv", r.snaps[:, 0].astype(np.float64), kh)
    rhs = (g * (1 - b * n2))[:, None] * np.einsum("hvk,hk->hv", S0.astype(np.float64), kh) \
        + (b * n2)[:, None] * v[:, 0]
    assert _relerr(lhs, rhs) < 1e-5


def _transition_form(S0, q, k, v, a, beta, scale):
    """S_t = g S_{t-1} (I - beta k k^T) + beta v k^T, o_t = S_t q_hat scale, in
    fp64 with matrix products (the same rule, written another way)."""
    H, T, K = q.shape
    S = S0.astype(np.float64)
    outs, states = [], []
    eye = np.eye(K)
    for t in range(T):
        kh = _norm64(k[:, t])
        qh = _norm64(q[:, t]) * scale
        g = np.exp(a[:, t].astype(np.float64))
        b = beta[:, t].astype(np.float64)
        A = g[:, None, None] * (eye[None] - b[:, None, None] * kh[:, :, None] * kh[:, None, :])
        S = S @ A + b[:, None, None] * v[:, t].astype(np.float64)[:, :, None] * kh[:, None, :]
        outs.append(np.einsum("hvk,hk->hv", S, qh))
        states.append(S.copy())
    return np.stack(outs, 1), np.stack(states, 1)


@pytest.mark.parametrize("seed", [0, 1, 2])
@pytest.mark.parametrize("extreme", [False, True])
def test_matches_transition_matrix_form(seed, extreme):
    S0, q, k, v, a, beta = _inputs(seed, K=128, V=128, extreme=extreme)
    scale = 128 ** -0.5 if seed == 1 else 1.0
    o64, s64 = _transition_form(S0, q, k, v, a, beta, scale)
    w = np.full(3, 4, np.int32)
    r32 = oracle.native_heads(S0, w, q, k, v, a, beta, scale=scale, snaps=True)
    r64 = oracle.native_heads(S0, w, q, k, v, a, beta, scale=scale, snaps=True,
                              dtype=np.float64, eps=float(F32(oracle.EPS)))
    for t in range(4):
        assert _relerr(r32.o[:, t], o64[:, t]) < 1e-5
        assert _relerr(r32.snaps[:, t], s64[:, t]) < 1e-5
        assert _relerr(r64.o[:, t], o64[:, t]) < 1e-11
        assert _relerr(r64.snaps[:, t], s64[:, t]) < 1e-11


def test_onehot_query_reads_one_column_of_the_updated_state():
    """q = e_i: o[v] = S_t[v][i] * q_hat_i, a single product, so the output is
    bit-exact; it reads the state after the token's update."""
    S0, q, k, v, a, beta = _inputs(9, K=16, V=12)
    i = 5
    q[:] = 0
    q[:, :, i] = 1
    r = oracle.native_heads(S0, np.full(3, 4, np.int32), q, k, v, a, beta, snaps=True)
    qh = F32(1) * (F32(1) / np.sqrt(F32(1) + F32(oracle.EPS)))
    for t in range(4):
        want = (r.snaps[:, t, :, i] * qh).astype(F32)
        assert np.array_equal(r.o[:, t], want)


def test_onehot_key_updates_one_column():
    """k = e_j: columns other than j are only decayed; column j gets the write."""
    S0, q, k, v, a, beta = _inputs(10, K=16, V=12)
    j = 3
    k[:] = 0
    k[:, :, j] = 2
    r = oracle.native_heads(S0, np.full(3, 1, np.int32), q, k, v, a, beta, snaps=True)
    g = r.rec_g[:, 0][:, None, None]
    decayed = (S0 * g).astype(F32)
    others = [c for c in range(16) if c != j]
    assert np.array_equal(r.snaps[:, 0][:, :, others], decayed[:, :, others])
    kh = 2.0 / np.sqrt(4.0 + np.float64(F32(oracle.EPS)))
    u = decayed[:, :, j].astype(np.float64) * kh
    want = decayed[:, :, j] + beta[:, 0][:, None] * (v[:, 0] - u) * kh
    assert _relerr(r.snaps[:, 0][:, :, j], want) < 1e-6


def test_record_key_is_normalised_and_gate_is_exp():
    S0, q, k, v, a, beta = _inputs(11, K=128, V=128)
    r = oracle.native_heads(S0, np.full(3, 4, np.int32), q, k, v, a, beta)
    assert _relerr(r.rec_khat, _norm64(k)) < 3e-7
    g64 = np.exp(a.astype(np.float64))
    assert np.all(np.abs(r.rec_g - g64) <= np.spacing(r.rec_g.astype(F32)))


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_fp32_within_tolerance_of_fp64(seed):
    """The fp32 oracle's own rounding error is far inside the 1e-5 tolerance
    used against the GPU."""
    S0, q, k, v, a, beta = _inputs(seed, H=4, K=128, V=128, extreme=(seed == 2))
    w = np.full(4, 4, np.int32)
    r32 = oracle.native_heads(S0, w, q, k, v, a, beta, snaps=True)
    r64 = oracle.native_heads(S0, w, q, k, v, a, beta, snaps=True, dtype=np.float64)
    assert _relerr(r32.snaps, r64.snaps) < 2e-6
    assert _relerr(r32.o, r64.o) < 2e-6


def test_record_size_matches_page_growth():
    """The record per token and value head is V + K + 1 fp32 values; at
    K = V = 128 and 4 verify tokens that is 6.27% of a 64 KiB head, the "about
    6%" page growth the vLLM RecoverSSM PR reports (Purpose, note on FULL
    graphs)."""
    S0, q, k, v, a, beta = _inputs(12, H=1, K=128, V=128)
    r = oracle.native_heads(S0, np.full(1, 4, np.int32), q, k, v, a, beta)
    per_token = r.rec_delta.shape[2] + r.rec_khat.shape[2] + 1
    ratio = 4 * per_token * 4 / (128 * 128 * 4)
    assert per_token == 257
    assert 0.055 < ratio < 0.065


# --------------------------------------------------------------------------
# bf16 rounding
# --------------------------------------------------------------------------

def test_bf16_rne_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.normal(0, 1, 20000), rng.normal(0, 1e-3, 2000), rng.normal(0, 1e30, 2000),
        [0.0, -0.0, np.inf, -np.inf, 1.0, -1.0, 3.4e38, 1e-40, -1e-45],
    ]).astype(F32)
    bits = x.view(np.uint32)
    ties = ((bits & 0xFFFF0000) | 0x8000).astype(np.uint32).view(F32)   # exact halfway cases
    x = np.concatenate([x, ties[np.isfinite(ties)]])
    got = oracle.f32_to_bf16_rne(x)
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, want)
    back = oracle.bf16_to_f32(got)
    assert np.array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())
    nan = oracle.f32_to_bf16_rne(np.array([np.nan], F32))
    assert np.isnan(oracle.bf16_to_f32(nan)).all()


def test_bf16_ties_round_to_even():
    # 1 + 2^-8 is halfway between bf16 1.0 and 1.0078125 -> even (1.0)
    # 1 + 3*2^-8 is halfway between 1.0078125 and 1.015625 -> even (1.015625)
    x = np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8)], F32)
    got = oracle.bf16_to_f32(oracle.f32_to_bf16_rne(x))
    assert got.tolist() == [1.0, 1.015625, -1.0]


# --------------------------------------------------------------------------
# Align plan
# --------------------------------------------------------------------------

def _golden():
    with open(os.path.join(HERE, "golden", "align_cases.json")) as f:
        return json.load(f)


def test_align_plan_hand_worked_cases():
    gold = _golden()
    cases = gold["cases"]
    p0 = [c["p0"] for c in cases]
    n = [c["n"] for c in cases]
    table = np.tile(np.array(gold["table"], np.int32), (len(cases), 1))
    src, dst, bl, bs, err = oracle.align_plan(p0, n, table, gold["block"], 16)
    for i, c in enumerate(cases):
        assert (src[i], dst[i], bl[i], bs[i], err[i]) == \
            (c["src"], c["dst"], c["bnd_len"], c["bnd_slot"], 0), c["name"]


@pytest.mark.parametrize("block,T", [(4, 4), (8, 4), (16, 16), (64, 16), (64, 4)])
def test_align_plan_closed_form(block, T):
    """Exhaustive over the offset inside the block and n, against the closed
    form: src column (p0-1)//B, final column (p0+n-1)//B, first boundary after
    t_b = B - p0 % B tokens (B when p0 % B == 0), written iff t_b < n."""
    rows = []
    for m in (1, 2, 5):
        for r in range(block):
            for n in range(T + 1):
                p0 = m * block + r
                if p0 >= 1:
                    rows.append((p0, n))
    p0 = np.array([x[0] for x in rows], np.int32)
    n = np.array([x[1] for x in rows], np.int32)
    cols = 8
    table = np.tile((100 + 7 * np.arange(cols)).astype(np.int32), (len(rows), 1))
    src, dst, bl, bs, err = oracle.align_plan(p0, n, table, block, T)
    assert not err.any()
    col = lambda c: 100 + 7 * c   # noqa: E731
    for i, (pp, nn) in enumerate(rows):
        assert src[i] == col((pp - 1) // block)
        if nn == 0:
            assert (dst[i], bl[i], bs[i]) == (-1, 0, -1)
            continue
        assert dst[i] == col((pp + nn - 1) // block)
        tb = block - pp % block if pp % block else block
        if tb < nn:
            assert (bl[i], bs[i]) == (tb, col((pp + tb - 1) // block))
            assert (pp + bl[i]) % block == 0          # a boundary state covers whole blocks
            assert bs[i] == src[i] or pp % block == 0
        else:
            assert (bl[i], bs[i]) == (0, -1)


def test_align_plan_errors():
    table = np.tile(np.array([10, 11, -1], np.int32), (5, 1))
    p0 = np.array([0, 5, 6, 127, 60], np.int32)
    n = np.array([1, 9, 4, 2, 4], np.int32)   # row 3 needs the empty column 2
    src, dst, bl, bs, err = oracle.align_plan(p0, n, table, 64, 8)
    assert err.tolist() == [64, 4, 0, 16, 0]
    assert (src[0], dst[0]) == (-1, -1) and (src[3], dst[3]) == (-1, -1)
    # a window longer than a block crosses two boundaries: rejected
    t2 = np.array([[1, 2, 3, 4]], np.int32)
    _, _, _, _, err2 = oracle.align_plan([3], [9], t2, 4, 16)
    assert err2.tolist() == [8]


# ---- gates from raw inputs ---------------------------------------------------
# Reading (the pages print no formula for this step): log-gate =
# -exp(A_log) softplus(a + dt_bias) with softplus linear above 20, beta =
# sigmoid(b). The pins below fix that formula's pieces by closed forms,
# identities and the library's own softplus / sigmoid.

def test_raw_gates_closed_forms():
    # softplus(0) = ln 2 and exp(0) = 1: log-gate -ln 2, decay exactly 1/2 in fp64
    lg, be = oracle.raw_gates([[0.0]], [[0.0]], [0.0], [0.0], dtype=np.float64)
    assert lg[0, 0] == pytest.approx(-np.log(2.0), rel=1e-15, abs=0)
    assert be[0, 0] == 0.5
    # linear branch: a + dt_bias = 25 > 20 gives softplus = 25; A_log = ln 3 gives rate 3
    lg, _ = oracle.raw_gates([[20.0]], [[0.0]], [np.log(3.0)], [5.0], dtype=np.float64)
    assert lg[0, 0] == pytest.approx(-75.0, rel=1e-14)
    # the split point itself stays on the log branch: softplus(20) = 20 + log1p(e^-20)
    lg, _ = oracle.raw_gates([[20.0]], [[0.0]], [0.0], [0.0], dtype=np.float64)
    assert lg[0, 0] == pytest.approx(-(20.0 + np.log1p(np.exp(-20.0))), rel=1e-15)


def test_raw_gates_identities_and_library_forms():
    rng = np.random.default_rng(5)
    x = rng.uniform(-19.0, 19.0, (64, 1))
    b = rng.normal(0, 3, (64, 1))
    zero = np.zeros(1)
    lg_p, be_p = oracle.raw_gates(x, b, zero, zero, dtype=np.float64)
    lg_m, be_m = oracle.raw_gates(-x, -b, zero, zero, dtype=np.float64)
    # softplus(x) - softplus(-x) = x; sigmoid(b) + sigmoid(-b) = 1
    np.testing.assert_allclose(lg_m - lg_p, x, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(be_p + be_m, 1.0, rtol=0, atol=1e-15)
    # library forms: softplus(x) = logaddexp(0, x), sigmoid = 1 / (1 + exp(-b))
    np.testing.assert_allclose(-lg_p, np.logaddexp(0.0, x), rtol=1e-14)
    import scipy.special
    np.testing.assert_allclose(be_p, scipy.special.expit(b), rtol=1e-14)


def test_raw_gates_per_head_parameters():
    """Entry i uses the parameters of head i % HV: rates 1, 2, 4 scale the
    log-gate of heads 0, 1, 2, and dt_bias shifts the input of its own head."""
    a = np.full((3, 3), 0.5)
    A_log = np.log([1.0, 2.0, 4.0])
    lg, _ = oracle.raw_gates(a, np.zeros((3, 3)), A_log, np.zeros(3), dtype=np.float64)
    sp = np.logaddexp(0.0, 0.5)
    np.testing.assert_allclose(lg, -np.array([[1.0, 2.0, 4.0]] * 3) * sp, rtol=1e-14)
    lg, _ = oracle.raw_gates(np.zeros((2, 3)), np.zeros((2, 3)), np.zeros(3),
                             np.array([0.0, 1.0, -1.0]), dtype=np.float64)
    np.testing.assert_allclose(lg, -np.logaddexp(0.0, np.array([[0.0, 1.0, -1.0]] * 2)),
                               rtol=1e-14)


def test_raw_gates_fp32_close_to_fp64():
    rng = np.random.default_rng(6)
    a = rng.normal(size=(32, 8)).astype(F32)
    b = rng.normal(size=(32, 8)).astype(F32)
    A_log = np.log(rng.uniform(1, 16, 8)).astype(F32)
    dtb = rng.normal(-4, 1, 8).astype(F32)
    lg32, be32 = oracle.raw_gates(a, b, A_log, dtb)
    lg64, be64 = oracle.raw_gates(a, b, A_log, dtb, dtype=np.float64)
    np.testing.assert_allclose(lg32, lg64, rtol=4e-7)
    np.testing.assert_allclose(be32, be64, rtol=4e-7)


# ---- short-conv state (token-by-token decode) ---------------------------------

def test_conv_decode_hand_worked():
    """L_s = 3 rows of 2 channels, two inputs, worked by hand: each token drops
    the oldest row and appends its input."""
    state = np.array([[1, 2], [3, 4], [5, 6]], np.float32)
    x = np.array([[7, 8], [9, 10]], np.float32)
    walk = oracle.conv_decode(state, x)
    np.testing.assert_array_equal(walk[0], state)
    np.testing.assert_array_equal(walk[1], [[3, 4], [5, 6], [7, 8]])
    np.testing.assert_array_equal(walk[2], [[5, 6], [7, 8], [9, 10]])
    fin, bnd = oracle.conv_commit(state, x, 2, bnd_len=1)
    np.testing.assert_array_equal(fin, walk[2])
    np.testing.assert_array_equal(bnd, walk[1])
    assert oracle.conv_commit(state, x, 2, bnd_len=2)[1] is None   # boundary at n: none


@pytest.mark.parametrize("Ls", [1, 3, 12])
def test_conv_decode_is_a_sliding_window(Ls):
    """After n tokens the state is rows n .. n+Ls-1 of [state; x] (closed
    form of the window), for n below and above L_s; n = 0 keeps the state;
    decoding in two pieces equals decoding at once."""
    rng = np.random.default_rng(Ls)
    state = rng.normal(size=(Ls, 8)).astype(np.float32)
    x = rng.normal(size=(Ls + 6, 8)).astype(np.float32)
    seq = np.concatenate([state, x])
    walk = oracle.conv_decode(state, x)
    for n in range(len(x) + 1):
        np.testing.assert_array_equal(walk[n], seq[n:n + Ls])
    np.testing.assert_array_equal(oracle.conv_commit(state, x, 0)[0], state)
    a = 4
    mid = oracle.conv_decode(state, x[:a])[a]
    np.testing.assert_array_equal(oracle.conv_decode(mid, x[a:])[-1], walk[-1])


# --------------------------------------------------------------------------
# The per-key-channel decay variant (the KDA reading)
# --------------------------------------------------------------------------

def _channel_a(seed, H, T, K, extreme=False):
    rng = np.random.default_rng(1000 + seed)
    a = (-np.logaddexp(0, rng.normal(size=(H, T, K)))).astype(F32)
    if extreme:
        a[:, 0, : K // 2] = 0.0      # no decay on half of the channels
        a[:, 1, K // 2:] = -100.0    # decay to the subnormal range on the others
    return a


@pytest.mark.parametrize("seed", [0, 1, 2])
@pytest.mark.parametrize("extreme", [False, True])
def test_channel_uniform_decay_is_the_scalar_rule(seed, extreme):
    """One decay repeated over every key channel gives the scalar rule's
    outputs, records and states bit for bit (fp32 and fp64)."""
    S0, q, k, v, a, beta = _inputs(seed, K=32, V=24, extreme=extreme)
    w = np.array([4, 3, 1], np.int32)
    ach = np.repeat(a[:, :, None], 32, 2)
    for dt in (np.float32, np.float64):
        r = oracle.native_heads(S0, w, q, k, v, a, beta, snaps=True, dtype=dt)
        c = oracle.native_heads_ch(S0, w, q, k, v, ach, beta, snaps=True, dtype=dt)
        for x, y in ((r.o, c.o), (r.rec_delta, c.rec_delta), (r.rec_khat, c.rec_khat),
                     (r.snaps, c.snaps), (np.repeat(r.rec_g[:, :, None], 32, 2), c.rec_alpha)):
            assert np.array_equal(x, y)


@pytest.mark.parametrize("seed", [0, 1, 2])
@pytest.mark.parametrize("K,V,T", [(4, 4, 4), (16, 12, 5), (128, 128, 4)])
def test_channel_replay_equals_native_state(seed, K, V, T):
    S0, q, k, v, _, beta = _inputs(seed, H=2, T=T, K=K, V=V)
    a = _channel_a(seed, 2, T, K)
    w = np.array([T, T - 2], np.int32)
    r = oracle.native_heads_ch(S0, w, q, k, v, a, beta, snaps=True)
    for h in range(2):
        for n in range(w[h] + 1):
            got = oracle.replay_heads_ch(S0[h:h + 1], [n], r.rec_delta[h:h + 1],
                                         r.rec_khat[h:h + 1], r.rec_alpha[h:h + 1])[0]
            want = S0[h] if n == 0 else r.snaps[h, n - 1]
            assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), (h, n)


def test_channel_no_write_decays_each_key_column():
    """beta = 0: S_t[v][k] = S_{t-1}[v][k] * alpha_t[k] exactly (columns are the
    key channels; a state scaled along its value rows instead fails)."""
    S0, q, k, v, _, beta = _inputs(5, K=16, V=16)
    a = _channel_a(5, 3, 4, 16)
    beta[:] = 0
    r = oracle.native_heads_ch(S0, np.full(3, 4, np.int32), q, k, v, a, beta, snaps=True)
    S = S0.copy()
    for t in range(4):
        al = r.rec_alpha[:, t]
        S = (S * al[:, None, :]).astype(F32)
        assert np.array_equal(r.snaps[:, t], S)
    rows_scaled = (S0 * r.rec_alpha[:, 0][:, :, None]).astype(F32)
    assert not np.array_equal(r.snaps[:, 0], rows_scaled)
    assert np.array_equal(r.rec_delta, np.zeros_like(r.rec_delta))


def _channel_transition_form(S0, q, k, v, a, beta, scale):
    """S_t = S_{t-1} Diag(alpha_t) (I - beta k k^T) + beta v k^T in fp64."""
    H, T, K = q.shape
    S = S0.astype(np.float64)
    outs, states = [], []
    eye = np.eye(K)
    for t in range(T):
        kh = _norm64(k[:, t])
        qh = _norm64(q[:, t]) * scale
        al = np.exp(a[:, t].astype(np.float64))
        b = beta[:, t].astype(np.float64)
        P = eye[None] - b[:, None, None] * kh[:, :, None] * kh[:, None, :]
        S = (S * al[:, None, :]) @ P + b[:, None, None] * v[:, t].astype(np.float64)[:, :, None] * kh[:, None, :]
        outs.append(np.einsum("hvk,hk->hv", S, qh))
        states.append(S.copy())
    return np.stack(outs, 1), np.stack(states, 1)


@pytest.mark.parametrize("seed", [0, 1])
@pytest.mark.parametrize("extreme", [False, True])
def test_channel_matches_transition_matrix_form(seed, extreme):
    S0, q, k, v, _, beta = _inputs(seed, K=128, V=128)
    a = _channel_a(seed, 3, 4, 128, extreme=extreme)
    o64, s64 = _channel_transition_form(S0, q, k, v, a, beta, 1.0)
    w = np.full(3, 4, np.int32)
    r32 = oracle.native_heads_ch(S0, w, q, k, v, a, beta, snaps=True)
    r64 = oracle.native_heads_ch(S0, w, q, k, v, a, beta, snaps=True, dtype=np.float64,
                                 eps=float(F32(oracle.EPS)))
    for t in range(4):
        assert _relerr(r32.o[:, t], o64[:, t]) < 1e-5
        assert _relerr(r32.snaps[:, t], s64[:, t]) < 1e-5
        assert _relerr(r64.o[:, t], o64[:, t]) < 1e-11
        assert _relerr(r64.snaps[:, t], s64[:, t]) < 1e-11


def test_channel_record_decay_is_exp():
    S0, q, k, v, _, beta = _inputs(12, K=128, V=128)
    a = _channel_a(12, 3, 4, 128)
    r = oracle.native_heads_ch(S0, np.full(3, 4, np.int32), q, k, v, a, beta)
    al64 = np.exp(a.astype(np.float64))
    assert np.all(np.abs(r.rec_alpha - al64) <= np.spacing(r.rec_alpha.astype(F32)))
    assert r.rec_g is None
