"""Independent fp64 formulations used to pin the oracle (test-only; imports nothing from the oracle).

Each function computes the same quantity as an oracle entry point by a *different* route, so that
a dropped term, a wrong sign, a wrong index or a transposed operand in the oracle shows up as a
disagreement:

* conv via ``numpy.correlate`` over the sequence extended by its carried window, with the kernel
  dilated by inserting zeros;
* the recurrence in matrix form ``S_t = g_t S_{t-1} (I - b_t k_t k_t^T) + b_t v_t k_t^T`` over the
  whole V x K state at once (the oracle runs one value column at a time);
* the recurrence in chunked WY / UT-transform form (chunk-parallel algebra; see ``chunked_wy``).
"""
from __future__ import annotations

import numpy as np
from scipy.special import expit


def conv_correlate(x_seq: np.ndarray, window: np.ndarray, w: np.ndarray, D: int, bias=None, silu=False):
    """One sequence, all channels.  x_seq [len, C], window [C, L], w [C, W] (float64).
    Returns (y [len, C], new_window [C, L])."""
    length, C = x_seq.shape
    W = w.shape[1]
    L = (W - 1) * D
    ext = np.concatenate([window.T, x_seq], axis=0)  # [L + len, C]
    y = np.zeros((length, C))
    for c in range(C if length > 0 else 0):
        kd = np.zeros(L + 1)
        kd[np.arange(W) * D] = w[c]  # dilated kernel: tap j sits at offset j*D
        y[:, c] = np.correlate(ext[:, c], kd, mode="valid")
    if bias is not None:
        y = y + bias[None, :]
    if silu:
        y = y * expit(y)
    new_window = ext[ext.shape[0] - L:, :].T if L > 0 else np.zeros((C, 0))
    return y, new_window


def l2n(x: np.ndarray) -> np.ndarray:
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + 1e-12)


def gates(a, b, A_log, dt_bias, *, softplus, sigmoid, T, H):
    """(g [T,H], beta [T,H]) in float64 from float inputs (None = absent)."""
    if a is None:
        g = np.ones((T, H))
    elif softplus:
        g = np.exp(-np.exp(A_log.astype(np.float64))[None, :] * np.logaddexp(a + dt_bias[None, :], 0.0))
    else:
        g = np.exp(a)
    if b is None:
        beta = np.ones((T, H))
    else:
        beta = expit(b) if sigmoid else b.copy()
    return g, beta


def matrix_form(qh, kh, g, beta, v, S0, scale):
    """One (sequence, head).  qh, kh [T,K]; g, beta [T]; v [T,V]; S0 [V,K].  Returns (o [T,V], S)."""
    T, K = kh.shape
    S = S0.copy()
    o = np.zeros((T, v.shape[1]))
    I = np.eye(K)
    for t in range(T):
        k = kh[t]
        S = g[t] * S @ (I - beta[t] * np.outer(k, k)) + beta[t] * np.outer(v[t], k)
        o[t] = scale * S @ qh[t]
    return o, S


def chunked_wy(qh, kh, g, beta, v, S0, scale, chunk):
    """Chunked WY form.  Within a chunk with local cumulative log-decay G_i = sum_{j<=i} log g_j:
    A_ij = b_i e^{G_i-G_j} (k_i.k_j) for j<i, T = (I+A)^{-1}, W = T diag(b e^G) K, U' = T diag(b) V,
    U = U' - W S0^T, O = scale [diag(e^G) Q S0^T + (M o QK^T) U] with M_ij = e^{G_i-G_j} (j<=i),
    S_end = e^{G_C} S0 + U^T diag(e^{G_C - G}) K.  Requires g > 0."""
    T, K = kh.shape
    S = S0.copy()
    o = np.zeros((T, v.shape[1]))
    for c0 in range(0, T, chunk):
        sl = slice(c0, min(c0 + chunk, T))
        Q, Kc, Vc, bc = qh[sl], kh[sl], v[sl], beta[sl]
        n = Kc.shape[0]
        G = np.cumsum(np.log(g[sl]))
        dG = G[:, None] - G[None, :]
        A = np.tril(bc[:, None] * np.exp(np.minimum(dG, 0.0)) * (Kc @ Kc.T), -1)
        Tm = np.linalg.inv(np.eye(n) + A)
        Wm = Tm @ ((bc * np.exp(G))[:, None] * Kc)
        Up = Tm @ (bc[:, None] * Vc)
        U = Up - Wm @ S.T
        M = np.tril(np.exp(np.minimum(dG, 0.0)))
        o[sl] = scale * (np.exp(G)[:, None] * (Q @ S.T) + (M * (Q @ Kc.T)) @ U)
        S = np.exp(G[-1]) * S + U.T @ (np.exp(G[-1] - G)[:, None] * Kc)
    return o, S
