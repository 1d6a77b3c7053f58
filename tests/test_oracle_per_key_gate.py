"""Pins for the oracle's per-key-channel decay (CPU only): the GatedDeltaNet thunk's
gate_per_channel form on the rlx-cpu thunk/types.rs page, where the decay input has one value per
key channel and the state's key axis decays channel by channel, S <- S diag(g) (I - beta k k^T) +
beta v k^T.

The pins: equal channel decays reproduce the per-head gate exactly; the column recurrence equals
that matrix form written out in numpy (GQA, softplus and raw decays, with and without the
retrieval term); a zero rate leaves pure channel-wise decay, a cumulative product; orthonormal keys
recall each value decayed by the later decays of its own channel only."""
import numpy as np
import pytest

import oracle
from forms import l2n
from test_oracle_scan import pack, rand_problem


def channel_gates(a, A_log, dtb, softplus):
    """g [T,H,K] from a [T,H,K] (A_log, dt_bias per head)."""
    a = a.astype(np.float64)
    if not softplus:
        return np.exp(a)
    return np.exp(-np.exp(A_log.astype(np.float64))[None, :, None] *
                  np.logaddexp(a + dtb.astype(np.float64)[None, :, None], 0.0))


def run(p, HQ, H, K, V, a, **kw):
    return oracle.scan(pack(p["q"], p["k"], p["v"]), p["off"], HQ=HQ, H=H, K=K, V=V, qkv_dtype="f32", a=a,
                       b=kw.pop("b", p["b"]), A_log=p["A_log"], dt_bias=p["dtb"], state_in=kw.pop("S0", p["S0"]),
                       **kw)


def test_equal_channel_decays_reduce_to_the_head_gate():
    HQ, H, K, V = 2, 4, 8, 5
    p = rand_problem(61, [7, 0, 4, 11], HQ, H, K, V)
    a_pk = np.ascontiguousarray(np.repeat(p["a"][:, :, None], K, axis=2))
    o1, s1 = run(p, HQ, H, K, V, p["a"])
    o2, s2 = run(p, HQ, H, K, V, a_pk, gate_per_key=True)
    assert np.array_equal(o1, o2) and np.array_equal(s1, s2)


@pytest.mark.parametrize("softplus", [True, False])
@pytest.mark.parametrize("retrieve", [True, False])
def test_matches_matrix_form_with_channel_decay(softplus, retrieve):
    HQ, H, K, V = 2, 4, 8, 5
    lengths = [9, 0, 5, 12]
    p = rand_problem(62, lengths, HQ, H, K, V)
    rng = np.random.default_rng(63)
    a_pk = rng.standard_normal((p["N"], H, K)).astype(np.float32)
    if not softplus:
        a_pk = rng.uniform(-1.0, 0.0, (p["N"], H, K)).astype(np.float32)
    out, st = run(p, HQ, H, K, V, a_pk, gate_per_key=True, softplus=softplus, retrieve=retrieve)
    g = channel_gates(a_pk, p["A_log"], p["dtb"], softplus)
    beta = 1.0 / (1.0 + np.exp(-p["b"].astype(np.float64)))
    qh, kh = l2n(p["q"].astype(np.float64)), l2n(p["k"].astype(np.float64))
    scale = 1.0 / np.sqrt(K)
    G = H // HQ
    I = np.eye(K)
    for i in range(len(lengths)):
        s0, s1 = p["off"][i], p["off"][i + 1]
        for h in range(H):
            S = p["S0"][i, h].astype(np.float64)
            for t in range(s0, s1):
                k = kh[t, h // G]
                P = I - beta[t, h] * np.outer(k, k) if retrieve else I
                S = S @ np.diag(g[t, h]) @ P + beta[t, h] * np.outer(p["v"][t, h], k)
                np.testing.assert_allclose(out[t, h], scale * S @ qh[t, h // G], rtol=1e-10, atol=1e-12)
            np.testing.assert_allclose(st[i, h], S, rtol=1e-10, atol=1e-12)


def test_zero_rate_is_pure_channel_decay():
    HQ, H, K, V = 1, 2, 8, 3
    p = rand_problem(64, [6, 3], HQ, H, K, V)
    a_pk = np.random.default_rng(65).standard_normal((p["N"], H, K)).astype(np.float32)
    zero = np.zeros_like(p["b"])
    out, st = run(p, HQ, H, K, V, a_pk, gate_per_key=True, b=zero, sigmoid=False)
    g = channel_gates(a_pk, p["A_log"], p["dtb"], True)
    qh = l2n(p["q"].astype(np.float64))
    for i in range(2):
        s0, s1 = p["off"][i], p["off"][i + 1]
        for h in range(H):
            cum = np.cumprod(g[s0:s1, h], axis=0)  # [T, K]
            S0 = p["S0"][i, h].astype(np.float64)
            for j, t in enumerate(range(s0, s1)):
                np.testing.assert_allclose(out[t, h], (S0 * cum[j][None, :]) @ qh[t, 0] / np.sqrt(K), rtol=1e-12)
            np.testing.assert_allclose(st[i, h], S0 * cum[-1][None, :], rtol=1e-12)


def test_orthonormal_keys_recall_with_channel_decay():
    K, V, T = 8, 4, 6
    rng = np.random.default_rng(66)
    q = np.zeros((T, 1, K), np.float32)
    k = np.zeros((T, 1, K), np.float32)
    for t in range(T):
        k[t, 0, t] = 1.0
    v = rng.standard_normal((T, 1, V)).astype(np.float32)
    a = rng.uniform(-1.0, 0.0, (T, 1, K)).astype(np.float32)
    p = dict(q=q, k=k, v=v, b=np.ones((T, 1), np.float32), off=np.array([0, T], np.int32), A_log=np.zeros(1, np.float32),
             dtb=np.zeros(1, np.float32), S0=None)
    _, st = run(p, 1, 1, K, V, a, gate_per_key=True, softplus=False, sigmoid=False)
    g = np.exp(a[:, 0].astype(np.float64))
    for j in range(T):
        np.testing.assert_allclose(st[0, 0][:, j], v[j, 0] * np.prod(g[j + 1:, j]), rtol=1e-12)
    assert not st[0, 0][:, T:].any()


def test_per_key_gate_is_not_combined_with_capture():
    p = rand_problem(67, [3], 1, 1, 8, 4)
    a_pk = np.zeros((p["N"], 1, 8), np.float32)
    with pytest.raises(ValueError):
        run(p, 1, 1, 8, 4, a_pk, gate_per_key=True, counts=np.array([2], np.int32), cap=2)
