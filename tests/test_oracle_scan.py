"""Pins for the oracle's gated delta-rule recurrence (CPU only).

The recurrence is the DELTA kernel string of the paged_ssm.rs page, per value column with a K-vector
state s: s <- g s; r = k.s; delta = beta (v - r); s <- s + delta k; o = scale q.s.  Each pin below
fixes it by something other than the oracle itself: an independent formulation (matrix form,
chunked WY form), exact rational arithmetic, closed forms of special cases, or invariances.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
import workloads
from forms import chunked_wy, gates, l2n, matrix_form


def pack(q, k, v):
    """q, k [N,HQ,K], v [N,H,V] float -> packed fp32 row [q | k | v]."""
    N = q.shape[0]
    flat = lambda x: x.reshape(N, int(np.prod(x.shape[1:])))
    return np.ascontiguousarray(np.concatenate([flat(q), flat(k), flat(v)], 1),
                                dtype=np.float32)


def rand_problem(seed, lengths, HQ, H, K, V, state=True):
    rng = np.random.default_rng(seed)
    off = workloads.offsets_from_lengths(lengths)
    N, B = int(off[-1]), len(lengths)
    q = rng.standard_normal((N, HQ, K)).astype(np.float32)
    k = rng.standard_normal((N, HQ, K)).astype(np.float32)
    v = rng.standard_normal((N, H, V)).astype(np.float32)
    a = rng.standard_normal((N, H)).astype(np.float32)
    b = rng.standard_normal((N, H)).astype(np.float32)
    A_log = rng.uniform(0, np.log(16), H).astype(np.float32)
    dtb = (rng.standard_normal(H) * 0.5).astype(np.float32)
    S0 = (rng.standard_normal((B, H, V, K)) * 0.1).astype(np.float32) if state else None
    return dict(off=off, q=q, k=k, v=v, a=a, b=b, A_log=A_log, dtb=dtb, S0=S0, N=N, B=B)


def run(p, HQ, H, K, V, scale=0.0, **kw):
    return oracle.scan(pack(p["q"], p["k"], p["v"]), p["off"], HQ=HQ, H=H, K=K, V=V, qkv_dtype="f32",
                       a=p["a"], b=p["b"], A_log=p["A_log"], dt_bias=p["dtb"], state_in=p["S0"], scale=scale, **kw)


@pytest.mark.parametrize("HQ,H", [(2, 2), (1, 3), (2, 4)])
def test_matches_matrix_form(HQ, H):
    K, V = 8, 5
    lengths = [9, 0, 4, 13]
    p = rand_problem(1, lengths, HQ, H, K, V)
    out, st = run(p, HQ, H, K, V)
    g, beta = gates(p["a"].astype(np.float64), p["b"].astype(np.float64), p["A_log"], p["dtb"].astype(np.float64),
                    softplus=True, sigmoid=True, T=p["N"], H=H)
    qh, kh = l2n(p["q"].astype(np.float64)), l2n(p["k"].astype(np.float64))
    G = H // HQ
    for i in range(len(lengths)):
        s, e = p["off"][i], p["off"][i + 1]
        for h in range(H):
            o_ref, S_ref = matrix_form(qh[s:e, h // G], kh[s:e, h // G], g[s:e, h], beta[s:e, h],
                                       p["v"][s:e, h].astype(np.float64), p["S0"][i, h].astype(np.float64),
                                       1 / np.sqrt(K))
            np.testing.assert_allclose(out[s:e, h], o_ref, rtol=1e-11, atol=1e-12)
            np.testing.assert_allclose(st[i, h], S_ref, rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("chunk", [1, 4, 64])
def test_matches_chunked_wy_form(chunk):
    HQ, H, K, V = 1, 2, 16, 8
    lengths = [150, 37]
    p = rand_problem(2, lengths, HQ, H, K, V)
    out, st = run(p, HQ, H, K, V)
    g, beta = gates(p["a"].astype(np.float64), p["b"].astype(np.float64), p["A_log"], p["dtb"].astype(np.float64),
                    softplus=True, sigmoid=True, T=p["N"], H=H)
    qh, kh = l2n(p["q"].astype(np.float64)), l2n(p["k"].astype(np.float64))
    for i in range(len(lengths)):
        s, e = p["off"][i], p["off"][i + 1]
        for h in range(H):
            o_ref, S_ref = chunked_wy(qh[s:e, 0], kh[s:e, 0], g[s:e, h], beta[s:e, h],
                                      p["v"][s:e, h].astype(np.float64), p["S0"][i, h].astype(np.float64),
                                      1 / np.sqrt(K), chunk)
            np.testing.assert_allclose(out[s:e, h], o_ref, rtol=1e-9, atol=1e-10)
            np.testing.assert_allclose(st[i, h], S_ref, rtol=1e-9, atol=1e-10)


def _exact_recurrence(q, k, v, g, beta, s0, scale):
    """Exact rational arithmetic for one column: lists of Fractions in, (outs, state) out."""
    s = list(s0)
    outs = []
    for t in range(len(v)):
        s = [g[t] * x for x in s]
        r = sum(ki * si for ki, si in zip(k[t], s))
        d = beta[t] * (v[t] - r)
        s = [si + d * ki for si, ki in zip(s, k[t])]
        outs.append(scale * sum(qi * si for qi, si in zip(q[t], s)))
    return outs, s


def test_brute_force_exact_rationals_tiny():
    # raw gates, no normalisation and dyadic inputs: the fp64 oracle must agree with exact arithmetic
    rng = np.random.default_rng(3)
    T, K, V = 6, 3, 2
    dy = lambda *s: (rng.integers(-8, 9, size=s) / 8.0).astype(np.float32)
    q, k, v = dy(T, 1, K), dy(T, 1, K), dy(T, 1, V)
    beta = (rng.integers(0, 9, size=(T, 1)) / 8.0).astype(np.float32)
    S0 = dy(1, 1, V, K)
    out, st = oracle.scan(pack(q, k, v), np.array([0, T], np.int32), HQ=1, H=1, K=K, V=V, qkv_dtype="f32",
                          b=beta, state_in=S0, l2norm=False, softplus=False, sigmoid=False, scale=0.5)
    F = lambda x: Fraction(float(x))
    for col in range(V):
        o, s = _exact_recurrence([[F(x) for x in q[t, 0]] for t in range(T)],
                                 [[F(x) for x in k[t, 0]] for t in range(T)],
                                 [F(v[t, 0, col]) for t in range(T)], [Fraction(1)] * T,
                                 [F(beta[t, 0]) for t in range(T)], [F(x) for x in S0[0, 0, col]], Fraction(1, 2))
        np.testing.assert_allclose(out[:, 0, col], [float(x) for x in o], rtol=1e-14, atol=1e-14)
        np.testing.assert_allclose(st[0, 0, col], [float(x) for x in s], rtol=1e-14, atol=1e-14)


def test_unit_gates_unit_key_retrieves_value_exactly():
    # g = 1, beta = 1, |k| = 1: after the write s.k == v, so q = k reads v back (scale 1), and
    # writing the same (k, v) again leaves the state unchanged.
    rng = np.random.default_rng(4)
    K, V = 8, 3
    k1 = np.zeros((1, 1, K), np.float32); k1[0, 0, 2] = 1.0
    ks = np.concatenate([k1, k1], 0)
    v1 = rng.standard_normal((1, 1, V)).astype(np.float32)
    vs = np.concatenate([v1, v1], 0)
    S0 = rng.standard_normal((1, 1, V, K)).astype(np.float32)
    out, st = oracle.scan(pack(ks, ks, vs), np.array([0, 2], np.int32), HQ=1, H=1, K=K, V=V, qkv_dtype="f32",
                          state_in=S0, l2norm=False, scale=1.0)
    np.testing.assert_allclose(out[:, 0], np.concatenate([v1[0], v1[0]]), rtol=1e-14, atol=1e-14)
    out1, st1 = oracle.scan(pack(k1, k1, v1), np.array([0, 1], np.int32), HQ=1, H=1, K=K, V=V, qkv_dtype="f32",
                            state_in=S0, l2norm=False, scale=1.0)
    np.testing.assert_allclose(st, st1, rtol=1e-14, atol=1e-14)


def test_zero_decay_resets_state():
    # g = exp(-inf) = 0: S_t = beta v k^T, o = scale beta v (k.q), independent of the past
    p = rand_problem(5, [6], 1, 2, 8, 4)
    a = np.full_like(p["a"], -np.inf)
    out, st = oracle.scan(pack(p["q"], p["k"], p["v"]), p["off"], HQ=1, H=2, K=8, V=4, qkv_dtype="f32", a=a,
                          b=p["b"], state_in=p["S0"], softplus=False, sigmoid=True, scale=0.0)
    qh, kh = l2n(p["q"].astype(np.float64)), l2n(p["k"].astype(np.float64))
    beta = 1 / (1 + np.exp(-p["b"].astype(np.float64)))
    for t in range(6):
        for h in range(2):
            want = beta[t, h] * p["v"][t, h] * (kh[t, 0] @ qh[t, 0]) / np.sqrt(8)
            np.testing.assert_allclose(out[t, h], want, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(st[0, 1], beta[5, 1] * np.outer(p["v"][5, 1], kh[5, 0]), rtol=1e-12, atol=1e-14)


def test_zero_rate_is_pure_decay():
    # beta = 0: o_t = scale e^{G_t} S0 q_t, final e^{G_T} S0
    HQ, H, K, V = 1, 2, 8, 4
    p = rand_problem(6, [10], HQ, H, K, V)
    b0 = np.zeros_like(p["b"])
    out, st = oracle.scan(pack(p["q"], p["k"], p["v"]), p["off"], HQ=HQ, H=H, K=K, V=V, qkv_dtype="f32", a=p["a"],
                          b=b0, A_log=p["A_log"], dt_bias=p["dtb"], state_in=p["S0"], sigmoid=False)
    g, _ = gates(p["a"].astype(np.float64), None, p["A_log"], p["dtb"].astype(np.float64), softplus=True,
                 sigmoid=False, T=10, H=H)
    G = np.cumprod(g, axis=0)
    qh = l2n(p["q"].astype(np.float64))
    for h in range(H):
        S0 = p["S0"][0, h].astype(np.float64)
        np.testing.assert_allclose(out[:, h], G[:, h:h + 1] * (qh[:, 0] @ S0.T) / np.sqrt(K), rtol=1e-12, atol=1e-15)
        np.testing.assert_allclose(st[0, h], G[-1, h] * S0, rtol=1e-12, atol=1e-15)


def test_linear_in_values_and_initial_state_jointly():
    HQ, H, K, V = 1, 1, 8, 4
    p = rand_problem(7, [12], HQ, H, K, V)
    rng = np.random.default_rng(70)
    dy = lambda *s: (rng.integers(-512, 512, size=s) / 128.0).astype(np.float32)  # sums exact in fp32
    v1, v2, S1, S2 = dy(12, 1, V), dy(12, 1, V), dy(1, 1, V, K), dy(1, 1, V, K)
    res = []
    for v, S in [(v1, S1), (v2, S2), (v1 + v2, S1 + S2)]:
        res.append(oracle.scan(pack(p["q"], p["k"], v), p["off"], HQ=HQ, H=H, K=K, V=V, qkv_dtype="f32", a=p["a"],
                               b=p["b"], A_log=p["A_log"], dt_bias=p["dtb"], state_in=S))
    np.testing.assert_allclose(res[2][0], res[0][0] + res[1][0], rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(res[2][1], res[0][1] + res[1][1], rtol=1e-11, atol=1e-12)


def test_split_and_carry_matches_single_call():
    HQ, H, K, V = 1, 2, 8, 4
    p = rand_problem(8, [17], HQ, H, K, V)
    full_o, full_s = run(p, HQ, H, K, V)
    for m in [0, 1, 9, 17]:
        sub = lambda sl: dict(p, q=p["q"][sl], k=p["k"][sl], v=p["v"][sl], a=p["a"][sl], b=p["b"][sl])
        o1, s1 = run(dict(sub(slice(0, m)), off=np.array([0, m], np.int32)), HQ, H, K, V)
        # the fp64 carried state is rounded to the fp32 state format between the two calls
        p2 = dict(sub(slice(m, 17)), off=np.array([0, 17 - m], np.int32), S0=s1.astype(np.float32))
        o2, s2 = run(p2, HQ, H, K, V)
        np.testing.assert_allclose(np.concatenate([o1, o2]), full_o, rtol=1e-5, atol=1e-6)
        np.testing.assert_allclose(s2, full_s, rtol=1e-5, atol=1e-6)


def test_sequence_permutation_invariance():
    HQ, H, K, V = 1, 2, 8, 4
    lengths = [5, 0, 9, 3]
    p = rand_problem(9, lengths, HQ, H, K, V)
    out, st = run(p, HQ, H, K, V)
    perm = [2, 0, 3, 1]
    off = p["off"]
    idx = np.concatenate([np.arange(off[i], off[i + 1]) for i in perm]).astype(np.int64)
    pp = dict(p, q=p["q"][idx], k=p["k"][idx], v=p["v"][idx], a=p["a"][idx], b=p["b"][idx], S0=p["S0"][perm],
              off=workloads.offsets_from_lengths([lengths[i] for i in perm]))
    out_p, st_p = run(pp, HQ, H, K, V)
    assert np.array_equal(out_p, out[idx])
    assert np.array_equal(st_p, st[perm])


def test_gqa_equals_duplicated_key_heads():
    HQ, H, K, V = 2, 6, 8, 4
    p = rand_problem(10, [7, 5], HQ, H, K, V)
    out, st = run(p, HQ, H, K, V)
    G = H // HQ
    rep = np.repeat(np.arange(HQ), G)  # value head h reads key head h // G
    pd = dict(p, q=p["q"][:, rep], k=p["k"][:, rep])
    out_d, st_d = run(pd, H, H, K, V)
    assert np.array_equal(out_d, out)
    assert np.array_equal(st_d, st)
    # and not the modulo mapping: a different grouping gives a different answer
    pm = dict(p, q=p["q"][:, np.arange(H) % HQ], k=p["k"][:, np.arange(H) % HQ])
    assert not np.allclose(run(pm, H, H, K, V)[0], out)


def test_scalar_closed_form_k1_v1():
    # K = V = 1 without normalisation: s <- g s (1 - beta k^2) + beta v k, o = scale q s
    rng = np.random.default_rng(11)
    T = 9
    q, k, v = (rng.standard_normal((T, 1, 1)).astype(np.float32) for _ in range(3))
    a = rng.uniform(-1, 0, (T, 1)).astype(np.float32)
    b = rng.uniform(0, 1, (T, 1)).astype(np.float32)
    s0 = np.array([[[[0.7]]]], np.float32)
    out, st = oracle.scan(pack(q, k, v), np.array([0, T], np.int32), HQ=1, H=1, K=1, V=1, qkv_dtype="f32", a=a, b=b,
                          state_in=s0, l2norm=False, softplus=False, sigmoid=False, scale=1.0)
    s = float(s0[0, 0, 0, 0])  # the fp32 value of 0.7
    for t in range(T):
        g, be, kk = np.exp(float(a[t, 0])), float(b[t, 0]), float(k[t, 0, 0])
        s = g * s * (1 - be * kk * kk) + be * float(v[t, 0, 0]) * kk
        assert out[t, 0, 0] == pytest.approx(float(q[t, 0, 0]) * s, rel=1e-13, abs=1e-15)
    assert st[0, 0, 0, 0] == pytest.approx(s, rel=1e-13)


def test_orthonormal_keys_store_and_recall_exactly():
    # keys e_0..e_{K-1}, g = beta = 1, zero state: S e_i = v_i; then query e_j reads v_j back
    K, V = 6, 3
    rng = np.random.default_rng(12)
    E = np.eye(K, dtype=np.float32)
    vals = rng.standard_normal((K, 1, V)).astype(np.float32)
    k = np.concatenate([E, E])[:, None, :]
    q = np.concatenate([E, E[::-1]])[:, None, :]
    v = np.concatenate([vals, vals])
    out, st = oracle.scan(pack(q, k, v), np.array([0, 2 * K], np.int32), HQ=1, H=1, K=K, V=V, qkv_dtype="f32",
                          l2norm=False, scale=1.0)
    assert np.array_equal(out[K:, 0], vals[::-1, 0].astype(np.float64))
    assert np.array_equal(st[0, 0], vals[:, 0].T.astype(np.float64))


def test_zero_length_sequences_copy_state_and_null_state_is_zero():
    HQ, H, K, V = 1, 1, 4, 2
    p = rand_problem(13, [0, 3, 0], HQ, H, K, V)
    _, st = run(p, HQ, H, K, V)
    assert np.array_equal(st[0], p["S0"][0].astype(np.float64))
    assert np.array_equal(st[2], p["S0"][2].astype(np.float64))
    o0, s0 = run(dict(p, S0=np.zeros_like(p["S0"])), HQ, H, K, V)
    o1, s1 = run(dict(p, S0=None), HQ, H, K, V)
    assert np.array_equal(o0, o1) and np.array_equal(s0, s1)


def test_malformed_offsets_write_nothing():
    p = rand_problem(14, [4, 5, 6, 2], 1, 1, 4, 2)
    for name, bad in workloads.malformed_offsets(p["off"]):
        assert run(dict(p, off=bad), 1, 1, 4, 2) is None, name


def test_default_scale_is_inverse_sqrt_k():
    p = rand_problem(15, [5], 1, 1, 16, 2)
    o_def, _ = run(p, 1, 1, 16, 2, scale=0.0)
    o_one, _ = run(p, 1, 1, 16, 2, scale=1.0)
    np.testing.assert_allclose(o_def, o_one / 4.0, rtol=1e-15)


def test_scale_zero_selects_inverse_sqrt_k_and_other_values_apply():
    """The host fn delta() substitutes 1/sqrt(K) for a zero scale attribute only: any other value,
    negative included, multiplies the readout.  The state never depends on the scale."""
    HQ, H, K, V = 1, 2, 16, 6
    p = rand_problem(7, [11, 5, 0], HQ, H, K, V)
    o0, s0 = run(p, HQ, H, K, V, scale=0.0)
    o1, s1 = run(p, HQ, H, K, V, scale=1.0)
    on, sn = run(p, HQ, H, K, V, scale=-0.375)
    op, sp = run(p, HQ, H, K, V, scale=0.375)
    assert np.allclose(o0, o1 / np.sqrt(K), rtol=1e-12, atol=0)
    assert np.array_equal(on, -op)
    for s in (s1, sn, sp):
        assert np.array_equal(s, s0)
