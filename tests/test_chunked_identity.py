"""The verify kernel evaluates the window through the unrolled recurrence
(no S_t is ever formed):
    u_p = G(0,p+1)(S0 k_p) + sum_{j<p}  G(j+1,p+1)(k_j . k_p) delta_j
    o_p = G(0,p+1)(S0 q_p) + sum_{j<=p} G(j+1,p+1)(k_j . q_p) delta_j
with G(a,b) the product of the gates a..b-1. This CPU test checks the identity
in fp64 against the per-token rule, ring prefixes and zero gates included."""
import numpy as np
import pytest


def _norm(x):
    return x / np.sqrt((x * x).sum() + 1e-6)


@pytest.mark.parametrize("seed", range(5))
def test_unrolled_recurrence_equals_per_token_rule(seed):
    rng = np.random.default_rng(seed)
    K = V = 16
    for trial in range(40):
        j0, w = int(rng.integers(0, 6)), int(rng.integers(1, 6))
        P = j0 + w
        S0 = rng.normal(0, .05, (V, K))
        kh = [_norm(rng.normal(size=K)) for _ in range(P)]
        qt = [_norm(rng.normal(size=K)) * 0.7 for _ in range(P)]
        v = [rng.normal(size=V) for _ in range(P)]
        g = np.exp(-np.log1p(np.exp(rng.normal(size=P))))
        if trial % 5 == 0:
            g[rng.integers(0, P)] = 0.0
        be = 1 / (1 + np.exp(-rng.normal(size=P)))
        h = S0.copy()
        d_ref, o_ref = [], []
        for p in range(P):                       # the per-token rule
            hp = g[p] * h
            d = be[p] * (v[p] - hp @ kh[p])
            h = hp + np.outer(d, kh[p])
            d_ref.append(d)
            o_ref.append(h @ qt[p])

        def G(a, b):
            return float(np.prod(g[a:b])) if b > a else 1.0
        d_ch = list(d_ref[:j0])                  # ring positions: recorded corrections
        for p in range(j0, P):
            u = G(0, p + 1) * (S0 @ kh[p]) + sum(G(j + 1, p + 1) * (kh[j] @ kh[p]) * d_ch[j]
                                                 for j in range(p))
            d = be[p] * (v[p] - u)
            d_ch.append(d)
            o = G(0, p + 1) * (S0 @ qt[p]) + sum(G(j + 1, p + 1) * (kh[j] @ qt[p]) * d_ch[j]
                                                 for j in range(p + 1))
            np.testing.assert_allclose(d, d_ref[p], rtol=1e-10, atol=1e-12)
            np.testing.assert_allclose(o, o_ref[p], rtol=1e-10, atol=1e-12)
