"""Pins for the oracle's update-rule switch (CPU only).

The pages' update_rule attribute compiles the DELTA kernel string with RETRIEVE = 0 for the
"linear" and "gated" rules: the write is delta = beta * v, with no retrieval term k.s (the decay
side of a rule is the presence of the decay input).  Without retrieval the recurrence is a
discounted sum, so each pin compares the oracle with that closed form, written independently of
the oracle's per-token loop:
    S_T = (prod_{t<=T} g_t) S_0 + sum_{t<=T} (prod_{t<u<=T} g_u) beta_t v_t k_t^T,   o_t = scale S_t q_t.
"""
import numpy as np
import pytest

import oracle
from forms import gates, l2n
from test_oracle_scan import pack, rand_problem


def closed_form(qh, kh, g, beta, v, S0, scale):
    """One sequence, one head: q, k [T,K]; g, beta [T]; v [T,V]; S0 [V,K] -> (o [T,V], S_T)."""
    T = qh.shape[0]
    o = np.zeros((T, v.shape[1]))
    logg = np.log(g)
    for t in range(T):
        # S_t = exp(sum_{u<=t} log g_u) S0 + sum_{j<=t} exp(sum_{j<u<=t} log g_u) beta_j v_j k_j^T
        w = np.exp(np.cumsum(logg[:t + 1][::-1])[::-1] - logg[:t + 1])  # prod_{j<u<=t} g_u, j = 0..t
        S = np.exp(logg[:t + 1].sum()) * S0 + np.einsum("j,jv,jk->vk", w * beta[:t + 1], v[:t + 1], kh[:t + 1])
        o[t] = scale * S @ qh[t]
    return o, S if T else S0


@pytest.mark.parametrize("decay", [False, True])
@pytest.mark.parametrize("HQ,H", [(1, 1), (2, 4)])
def test_no_retrieval_is_the_discounted_sum(decay, HQ, H):
    K, V = 6, 5
    lengths = [7, 0, 3, 11]
    p = rand_problem(11, lengths, HQ, H, K, V)
    if not decay:
        p["a"] = None
    # raw log-decays in [-1, 0] and sigmoid rates, L2-normalised q/k
    if decay:
        p["a"] = -np.abs(p["a"]) * 0.5
    out, st = oracle.scan(pack(p["q"], p["k"], p["v"]), p["off"], HQ=HQ, H=H, K=K, V=V, qkv_dtype="f32", a=p["a"],
                          b=p["b"], state_in=p["S0"], softplus=False, sigmoid=True, retrieve=False)
    g = np.exp(p["a"].astype(np.float64)) if decay else np.ones((p["N"], H))
    beta = 1.0 / (1.0 + np.exp(-p["b"].astype(np.float64)))
    qh, kh = l2n(p["q"].astype(np.float64)), l2n(p["k"].astype(np.float64))
    G = H // HQ
    scale = 1.0 / np.sqrt(K)
    for i in range(len(lengths)):
        s, e = p["off"][i], p["off"][i + 1]
        for h in range(H):
            o_ref, S_ref = closed_form(qh[s:e, h // G], kh[s:e, h // G], g[s:e, h], beta[s:e, h],
                                       p["v"][s:e, h].astype(np.float64), p["S0"][i, h].astype(np.float64), scale)
            np.testing.assert_allclose(out[s:e, h], o_ref, rtol=1e-9, atol=1e-12)
            np.testing.assert_allclose(st[i, h], S_ref, rtol=1e-9, atol=1e-12)


def test_retrieval_switch_changes_only_what_it_should():
    """beta = 0 writes nothing either way (pure decay); with writes, the two rules differ."""
    K, V, HQ, H = 8, 4, 2, 2
    p = rand_problem(12, [9, 5], HQ, H, K, V)
    b0 = np.full_like(p["b"], -1e4)  # sigmoid(-1e4) == 0 exactly in fp64 after the exp underflow
    kw = dict(HQ=HQ, H=H, K=K, V=V, qkv_dtype="f32", a=p["a"], A_log=p["A_log"], dt_bias=p["dtb"], state_in=p["S0"])
    qkv = pack(p["q"], p["k"], p["v"])
    o1, s1 = oracle.scan(qkv, p["off"], b=b0, retrieve=True, **kw)
    o2, s2 = oracle.scan(qkv, p["off"], b=b0, retrieve=False, **kw)
    assert np.array_equal(o1, o2) and np.array_equal(s1, s2)
    o3, _ = oracle.scan(qkv, p["off"], b=p["b"], retrieve=True, **kw)
    o4, _ = oracle.scan(qkv, p["off"], b=p["b"], retrieve=False, **kw)
    assert np.max(np.abs(o3 - o4)) > 1e-3


def test_gates_helper_is_consistent():
    """The gate helper the other pins use agrees with the raw-decay exponent used above."""
    a = np.array([[-0.25, -1.0]])
    g, _ = gates(a, np.zeros_like(a), None, None, softplus=False, sigmoid=False, T=1, H=2)
    np.testing.assert_allclose(g, np.exp(a))
