"""Pins for the oracle's varlen causal conv1d (CPU only).

The conv is fixed by the CONV kernel string of the paged_ssm.rs page: tap j of a width-W,
dilation-D filter reads token t-(W-1-j)*D, drawing on the carried window before the sequence
start; the new window is the last (W-1)*D entries of (old window ++ tokens).
"""
import numpy as np
import pytest

import oracle
import workloads
from forms import conv_correlate


def _case(seed, lengths, C, W, D, io="f32", state_dtype=None, bias=True, window=True):
    rng = np.random.default_rng(seed)
    state_dtype = state_dtype or io
    off = workloads.offsets_from_lengths(lengths)
    N, B, L = int(off[-1]), len(lengths), (W - 1) * D
    x = workloads.to_raw(rng.standard_normal((N, C)), io)
    w = workloads.to_raw(rng.standard_normal((C, W)) * 0.5, io)
    b = workloads.to_raw(rng.standard_normal(C) * 0.5, io) if bias else None
    st = workloads.to_raw(rng.standard_normal((B, C, L)), state_dtype) if (window and L > 0) else None
    return off, x, w, b, st


@pytest.mark.parametrize("W,D", [(4, 1), (3, 2), (2, 3), (1, 1), (5, 1)])
@pytest.mark.parametrize("silu", [False, True])
@pytest.mark.parametrize("io,sd", [("f32", "f32"), ("bf16", "f32"), ("f16", "f16")])
def test_conv_matches_numpy_correlate(W, D, silu, io, sd):
    lengths = [7, 0, 1, 3, 12]
    off, x, w, b, st = _case(1, lengths, C=6, W=W, D=D, io=io, state_dtype=sd)
    y, st_out = oracle.conv(x, w, off, W=W, D=D, x_dtype=io, bias=b, state_in=st, state_dtype=sd, silu=silu)
    xf = workloads.from_raw(x, io).astype(np.float64)
    wf = workloads.from_raw(w, io).astype(np.float64)
    bf = workloads.from_raw(b, io).astype(np.float64)
    L = (W - 1) * D
    for i in range(len(lengths)):
        s, e = off[i], off[i + 1]
        win = workloads.from_raw(st[i], sd).astype(np.float64) if st is not None else np.zeros((6, L))
        yr, wr = conv_correlate(xf[s:e], win, wf, D, bias=bf, silu=silu)
        np.testing.assert_allclose(y[s:e], yr, rtol=1e-13, atol=1e-13)
        assert np.array_equal(st_out[i], wr)  # the window is an exact copy


@pytest.mark.parametrize("W,D", [(4, 1), (3, 2)])
def test_delta_weight_is_identity_bit_exact(W, D):
    off, x, w, _, st = _case(2, [9, 2, 0, 5], C=8, W=W, D=D, io="bf16", bias=False)
    wd = np.zeros((8, W), np.float32)
    wd[:, W - 1] = 1.0
    y, _ = oracle.conv(x, workloads.to_raw(wd, "bf16"), off, W=W, D=D, x_dtype="bf16", state_in=st)
    assert np.array_equal(y, workloads.from_raw(x, "bf16").astype(np.float64))


@pytest.mark.parametrize("j", [0, 1, 2])
def test_single_tap_is_exact_shift_into_window(j):
    W, D = 3, 2
    L = (W - 1) * D
    off, x, _, _, st = _case(3, [6, 1, 3], C=4, W=W, D=D, io="f32", bias=False)
    wd = np.zeros((4, W), np.float32)
    wd[:, j] = 1.0
    y, _ = oracle.conv(x, wd, off, W=W, D=D, x_dtype="f32", state_in=st)
    for i in range(3):
        s, e = off[i], off[i + 1]
        for l in range(e - s):
            m = l - (W - 1 - j) * D
            want = x[s + m] if m >= 0 else st[i, :, L + m]
            assert np.array_equal(y[s + l], want.astype(np.float64))


def test_split_and_carry_matches_single_call():
    W, D = 4, 1
    off, x, w, b, st = _case(4, [20], C=5, W=W, D=D, io="f32")
    y_full, st_full = oracle.conv(x, w, off, W=W, D=D, x_dtype="f32", bias=b, state_in=st, silu=True)
    for m in [0, 1, 2, 3, 7, 20]:
        y1, st1 = oracle.conv(x[:m], w, np.array([0, m], np.int32), W=W, D=D, x_dtype="f32", bias=b,
                              state_in=st, silu=True)
        y2, st2 = oracle.conv(x[m:], w, np.array([0, 20 - m], np.int32), W=W, D=D, x_dtype="f32", bias=b,
                              state_in=st1.astype(np.float32), silu=True)
        assert np.array_equal(np.concatenate([y1, y2]), y_full)
        assert np.array_equal(st2, st_full)


def test_zero_length_sequences_copy_window_and_null_window_is_zero():
    off, x, w, b, st = _case(5, [0, 4, 0], C=3, W=4, D=1, io="f32")
    _, st_out = oracle.conv(x, w, off, W=4, D=1, x_dtype="f32", bias=b, state_in=st)
    assert np.array_equal(st_out[0], st[0].astype(np.float64))
    assert np.array_equal(st_out[2], st[2].astype(np.float64))
    y0, _ = oracle.conv(x, w, off, W=4, D=1, x_dtype="f32", bias=b, state_in=np.zeros_like(st))
    y1, _ = oracle.conv(x, w, off, W=4, D=1, x_dtype="f32", bias=b, state_in=None)
    assert np.array_equal(y0, y1)


def test_malformed_offsets_write_nothing():
    off, x, w, b, st = _case(6, [5, 6, 7, 8], C=3, W=4, D=1, io="f32")
    for name, bad in workloads.malformed_offsets(off):
        assert oracle.conv(x, w, bad, W=4, D=1, x_dtype="f32", bias=b, state_in=st) is None, name


def test_conv_is_linear_in_input_and_window_without_bias_and_activation():
    rng = np.random.default_rng(7)
    off = workloads.offsets_from_lengths([5, 3])
    # multiples of 2^-8 in [-4, 4): sums stay exact in fp32
    q = lambda *s: (rng.integers(-1024, 1024, size=s) / 256.0).astype(np.float32)
    x1, x2, s1, s2 = q(8, 4), q(8, 4), q(2, 4, 3), q(2, 4, 3)
    w = rng.standard_normal((4, 4)).astype(np.float32)
    ya, sa = oracle.conv(x1, w, off, W=4, D=1, x_dtype="f32", state_in=s1)
    yb, sb = oracle.conv(x2, w, off, W=4, D=1, x_dtype="f32", state_in=s2)
    yc, sc = oracle.conv(x1 + x2, w, off, W=4, D=1, x_dtype="f32", state_in=s1 + s2)
    np.testing.assert_allclose(yc, ya + yb, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(sc, sa + sb, rtol=0, atol=0)
