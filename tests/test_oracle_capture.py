"""Pins for the oracle's speculative-decoding capture (CPU only).

The pages record, per sequence, the first min(counts[b], cap, len) steps: the conv's raw token rows
(CONV_CAPTURE_*) and the recurrence's rank-1 updates (DELTA_CAPTURE_*): the decay g, the normalised
key k^ and the written value delta.  The pins: replaying the recorded updates from the initial
state gives the state an independent oracle run reaches after that many tokens; g and k^ equal
their definitions computed here; slots past the recorded count, an inactive step and
non-positive counts are zero; the conv record is the input rows."""
import numpy as np
import pytest

import oracle
import workloads
from forms import gates, l2n
from test_oracle_scan import pack, rand_problem

CAP = 4


def split(capsule, B, cap, HQ, H, K, V):
    g = capsule[:, :cap * H].reshape(B, cap, H)
    kh = capsule[:, cap * H:cap * (H + HQ * K)].reshape(B, cap, HQ, K)
    d = capsule[:, cap * (H + HQ * K):].reshape(B, cap, H, V)
    return g, kh, d


@pytest.mark.parametrize("retrieve", [True, False])
def test_replay_of_the_record_reaches_the_truncated_run_state(retrieve):
    HQ, H, K, V = 2, 4, 8, 5
    lengths = [6, 0, 3, 1, 9, 2]
    counts = np.array([3, 2, 8, 1, 0, -1], np.int32)
    p = rand_problem(31, lengths, HQ, H, K, V)
    qkv = pack(p["q"], p["k"], p["v"])
    kw = dict(HQ=HQ, H=H, K=K, V=V, qkv_dtype="f32", a=p["a"], b=p["b"], A_log=p["A_log"], dt_bias=p["dtb"],
              state_in=p["S0"], retrieve=retrieve)
    out, st, capsule = oracle.scan(qkv, p["off"], counts=counts, cap=CAP, **kw)
    g, khat, d = split(capsule, len(lengths), CAP, HQ, H, K, V)
    captured = np.clip(np.minimum(np.minimum(counts, CAP), lengths), 0, None)
    # independent run on every sequence cut to its recorded prefix
    tl = [int(c) for c in captured]
    toff = workloads.offsets_from_lengths(tl)
    rows = np.concatenate([np.arange(p["off"][i], p["off"][i] + tl[i]) for i in range(len(lengths))]).astype(int)
    sub = dict(kw, a=p["a"][rows], b=p["b"][rows])
    _, st_cut = oracle.scan(np.ascontiguousarray(qkv[rows]), toff, **sub)
    G = H // HQ
    for i in range(len(lengths)):
        for h in range(H):
            S = p["S0"][i, h].astype(np.float64)
            for j in range(captured[i]):
                S = g[i, j, h] * S + np.outer(d[i, j, h], khat[i, j, h // G])
            np.testing.assert_allclose(S, st_cut[i, h], rtol=1e-12, atol=1e-12)
        # slots past the record are zero
        assert not g[i, captured[i]:].any() and not khat[i, captured[i]:].any() and not d[i, captured[i]:].any()


def test_recorded_gates_and_keys_are_their_definitions():
    HQ, H, K, V = 2, 4, 8, 3
    lengths = [5, 4]
    p = rand_problem(32, lengths, HQ, H, K, V)
    _, _, capsule = oracle.scan(pack(p["q"], p["k"], p["v"]), p["off"], HQ=HQ, H=H, K=K, V=V, qkv_dtype="f32",
                                a=p["a"], b=p["b"], A_log=p["A_log"], dt_bias=p["dtb"], state_in=p["S0"],
                                counts=np.array([9, 9], np.int32), cap=CAP)
    g, khat, _ = split(capsule, 2, CAP, HQ, H, K, V)
    g_ref, _ = gates(p["a"].astype(np.float64), p["b"].astype(np.float64), p["A_log"], p["dtb"].astype(np.float64),
                     softplus=True, sigmoid=True, T=p["N"], H=H)
    kn = l2n(p["k"].astype(np.float64))
    for i in range(2):
        s = p["off"][i]
        np.testing.assert_allclose(g[i], g_ref[s:s + CAP], rtol=1e-12)
        np.testing.assert_allclose(khat[i], kn[s:s + CAP], rtol=1e-12)


def test_inactive_step_records_nothing():
    HQ, H, K, V = 1, 2, 8, 4
    p = rand_problem(33, [5, 3], HQ, H, K, V)
    kw = dict(HQ=HQ, H=H, K=K, V=V, qkv_dtype="f32", a=p["a"], b=p["b"], A_log=p["A_log"], dt_bias=p["dtb"],
              state_in=p["S0"], counts=np.array([4, 4], np.int32), cap=CAP)
    o1, s1, c1 = oracle.scan(pack(p["q"], p["k"], p["v"]), p["off"], active=np.array([0], np.int32), **kw)
    o2, s2, c2 = oracle.scan(pack(p["q"], p["k"], p["v"]), p["off"], active=np.array([1], np.int32), **kw)
    assert not c1.any() and c2.any()
    assert np.array_equal(o1, o2) and np.array_equal(s1, s2)  # recording never changes the result


@pytest.mark.parametrize("io", ["f32", "bf16", "f16"])
def test_conv_record_is_the_input_rows(io):
    w = workloads.make(name="cap_conv", seed=34, lengths=[3, 0, 7, 1], HQ=1, H=1, K=32, V=32, io=io)
    counts = np.array([5, 3, 2, 0], np.int32)
    upd = oracle.conv_capture(w.x, w.offsets, counts, cap=CAP, x_dtype=io)
    x = workloads.from_raw(w.x, io).astype(np.float64)
    for b in range(w.B):
        n = max(0, min(counts[b], CAP, w.lengths[b]))
        s = w.offsets[b]
        assert np.array_equal(upd[b, :n], x[s:s + n])
        assert not upd[b, n:].any()
    assert oracle.conv_capture(w.x, np.array([0, 3, 2, 10, 11], np.int32), counts, cap=CAP, x_dtype=io) is None
