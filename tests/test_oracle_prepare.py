"""Pins for the oracle's q/k normalisation and gate/rate activations (CPU only).

Definitions from the DELTA_PREPARE kernel string of the paged_ssm.rs page and the rate-activation
graph of the gated_delta_rate_activation.rs page: q and k are scaled by 1/sqrt(sum x^2 + 1e-12);
g = exp(-exp(A_log) * softplus(a + dt_bias)) or exp(a) for a raw log-decay; beta = sigmoid(b) or b.
"""
import math

import numpy as np
import pytest
from scipy.special import expit

import oracle
import workloads


def _qkv(seed, N, HQ, H, K, V, io="f32", scale=1.0):
    rng = np.random.default_rng(seed)
    return workloads.to_raw(rng.standard_normal((N, 2 * HQ * K + H * V)) * scale, io)


@pytest.mark.parametrize("io", ["f32", "bf16", "f16"])
def test_norm_closed_form_and_direction(io):
    N, HQ, H, K, V = 5, 2, 4, 16, 8
    qkv = _qkv(1, N, HQ, H, K, V, io, scale=3.0)
    qk, _ = oracle.prepare(qkv, HQ=HQ, H=H, K=K, V=V, qkv_dtype=io, l2norm=True)
    xf = workloads.from_raw(qkv, io).astype(np.float64)
    for plane in range(2):
        raw = xf[:, plane * HQ * K:(plane + 1) * HQ * K].reshape(N, HQ, K)
        nrm = np.linalg.norm(raw, axis=-1)
        np.testing.assert_allclose(np.linalg.norm(qk[plane], axis=-1), nrm / np.sqrt(nrm**2 + 1e-12), rtol=1e-14)
        # same direction: the normalised vector is a positive multiple of the input
        ratio = qk[plane] / raw
        np.testing.assert_allclose(ratio, ratio[..., :1] * np.ones_like(ratio), rtol=1e-13)
        assert np.all(ratio > 0)


def test_norm_epsilon_sits_inside_the_root():
    # a zero vector stays zero, a tiny vector is scaled by 1/sqrt(|x|^2 + 1e-12), not clamped
    N, HQ, H, K, V = 2, 1, 1, 4, 4
    x = np.zeros((N, 2 * K + V), np.float32)
    x[1, :K] = 1e-7
    qk, _ = oracle.prepare(x, HQ=HQ, H=H, K=K, V=V, qkv_dtype="f32", l2norm=True)
    assert np.all(qk[:, 0] == 0.0) and np.all(qk[1, 1] == 0.0)
    v = np.float64(np.float32(1e-7))
    np.testing.assert_allclose(qk[0, 1, 0], np.full(K, v / math.sqrt(K * v * v + 1e-12)), rtol=1e-14)


def test_norm_off_passes_values_through():
    N, HQ, H, K, V = 3, 2, 2, 8, 8
    qkv = _qkv(2, N, HQ, H, K, V, "f16")
    qk, _ = oracle.prepare(qkv, HQ=HQ, H=H, K=K, V=V, qkv_dtype="f16", l2norm=False)
    xf = workloads.from_raw(qkv, "f16").astype(np.float64)
    assert np.array_equal(qk[0], xf[:, :HQ * K].reshape(N, HQ, K))
    assert np.array_equal(qk[1], xf[:, HQ * K:2 * HQ * K].reshape(N, HQ, K))


def test_gate_closed_forms_at_zero_input():
    # softplus(0) = ln 2, so with a = dt_bias = 0: g = 2^(-exp(A_log)); A_log = 0 -> 1/2; sigmoid(0) = 1/2
    N, HQ, H, K, V = 1, 1, 3, 4, 4
    qkv = _qkv(3, N, HQ, H, K, V)
    A_log = np.array([0.0, math.log(16.0), math.log(3.0)], np.float32)
    z = np.zeros((N, H), np.float32)
    _, gb = oracle.prepare(qkv, HQ=HQ, H=H, K=K, V=V, qkv_dtype="f32", a=z, b=z, A_log=A_log,
                           dt_bias=np.zeros(H, np.float32))
    assert gb[0, 0, 0] == pytest.approx(0.5, rel=1e-15)
    np.testing.assert_allclose(gb[0, 0], 2.0 ** -np.exp(A_log.astype(np.float64)), rtol=1e-13)
    assert gb[0, 0, 1] == pytest.approx(2.0 ** -16, rel=1e-5)  # A_log = ln 16 rounded to fp32
    np.testing.assert_array_equal(gb[1, 0], 0.5)


def test_softplus_gate_matches_logaddexp_and_sigmoid_matches_expit():
    rng = np.random.default_rng(4)
    N, HQ, H, K, V = 50, 1, 4, 4, 4
    qkv = _qkv(4, N, HQ, H, K, V, "bf16")
    a = workloads.to_raw(rng.standard_normal((N, H)) * 20, "bf16")  # reaches both softplus tails
    b = workloads.to_raw(rng.standard_normal((N, H)) * 10, "bf16")
    A_log = rng.uniform(0, math.log(16), H).astype(np.float32)
    dtb = rng.standard_normal(H).astype(np.float32)
    _, gb = oracle.prepare(qkv, HQ=HQ, H=H, K=K, V=V, qkv_dtype="bf16", a=a, b=b, A_log=A_log, dt_bias=dtb)
    af = workloads.from_raw(a, "bf16").astype(np.float64)
    bf = workloads.from_raw(b, "bf16").astype(np.float64)
    want_g = np.exp(-np.exp(A_log.astype(np.float64)) * np.logaddexp(af + dtb.astype(np.float64), 0.0))
    np.testing.assert_allclose(gb[0], want_g, rtol=1e-12, atol=1e-300)
    np.testing.assert_allclose(gb[1], expit(bf), rtol=1e-14)
    assert np.all((gb[0] >= 0) & (gb[0] <= 1)) and np.all((gb[1] > 0) & (gb[1] < 1))


def test_raw_and_absent_gates():
    rng = np.random.default_rng(5)
    N, HQ, H, K, V = 7, 1, 2, 4, 4
    qkv = _qkv(5, N, HQ, H, K, V, "f16")
    a = workloads.to_raw(rng.uniform(-1, 0, (N, H)), "f16")
    b = workloads.to_raw(rng.uniform(0, 1, (N, H)), "f16")
    _, gb = oracle.prepare(qkv, HQ=HQ, H=H, K=K, V=V, qkv_dtype="f16", a=a, b=b, softplus=False, sigmoid=False)
    np.testing.assert_allclose(gb[0], np.exp(workloads.from_raw(a, "f16").astype(np.float64)), rtol=1e-15)
    assert np.array_equal(gb[1], workloads.from_raw(b, "f16").astype(np.float64))
    _, gb = oracle.prepare(qkv, HQ=HQ, H=H, K=K, V=V, qkv_dtype="f16")
    assert np.all(gb == 1.0)


def test_gate_inputs_may_be_fp32_with_half_qkv():
    rng = np.random.default_rng(6)
    N, HQ, H, K, V = 4, 1, 2, 4, 4
    qkv = _qkv(6, N, HQ, H, K, V, "bf16")
    a = rng.standard_normal((N, H)).astype(np.float32)
    A_log = np.zeros(H, np.float32)
    _, g32 = oracle.prepare(qkv, HQ=HQ, H=H, K=K, V=V, qkv_dtype="bf16", gate_dtype="f32", a=a, A_log=A_log,
                            dt_bias=np.zeros(H, np.float32))
    np.testing.assert_allclose(g32[0], np.exp(-np.logaddexp(a.astype(np.float64), 0.0)), rtol=1e-14)
