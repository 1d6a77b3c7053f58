"""Helpers for the GPU parity tests: moving seeded workloads to the device, slicing sampled
sub-problems for the oracle, and the error metric.  No arithmetic of the method lives here."""
from __future__ import annotations

import os

import numpy as np
import pytest

import workloads

TORCH_DT = {"f32": "float32", "bf16": "bfloat16", "f16": "float16"}
TOL = {"f32": 1e-4, "bf16": 2e-2, "f16": 2e-2}  # max relative error per output tensor
PREP_TOL = 1e-4  # fp32 prepare outputs from exactly decoded inputs
# fp32 final state of the token-sequential paths (DECODE, SEQ, the fused decode step): computed in
# fp32 from exactly decoded inputs whatever the I/O dtype, so fp32 accumulation bounds it; the
# chunked form rounds its operands to bf16 and keeps the I/O tolerance
SEQ_STATE_TOL = 1e-4
# a state downstream of a conv output that was rounded to bf16/fp16 (the chained decode step): the
# kernel's fp32 tap sum and the oracle's fp64 sum can round an element one unit apart, which moves
# the state by at most that unit relative to it (2^-8 for bf16)
CHAIN_STATE_TOL = 2.0 ** -8
# The chunked form runs its contractions on MFMA operands of the I/O type.  bf16 I/O: bf16 operands
# (8-bit significand), the half-precision bar of 2e-2.  fp16 I/O: fp16 operands (11-bit
# significand); each of the chain's roundings (q, k, S, R, T, U, P and the output) is then at most
# 2^-12 relative and together they stay near 1e-3 normwise, gated at 1.5e-3 (chunked against SEQ,
# which carries its own output rounding: 2e-3).
CHUNK_TOL = {"bf16": 2e-2, "f16": 1.5e-3}
CHUNK_SEQ_TOL = {"bf16": 2e-2, "f16": 2e-3}
# per (sequence, head) slice, the operand rounding is relative to the slice's intermediate terms,
# not its (possibly smaller) outputs
CHUNK_SLICE_TOL = {"bf16": 5e-2, "f16": 3e-3}


def state_tol(io: str, path: str) -> float:
    return CHUNK_TOL[io] if path == "chunk" else SEQ_STATE_TOL


def out_tol(io: str, path: str) -> float:
    return CHUNK_TOL[io] if path == "chunk" else TOL[io]


# achieved errors of this process's comparisons (test id, what, normwise, elementwise, gate); written
# as JSON lines at the end of the session when GDN_ERR_LOG names a file
RECORD: list = []


def require_gpu():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_delta_rule_varlen_amd as gdn  # noqa: F401  (fails loudly when libgdn.so is missing)

    return torch


def ensure_built():
    """Build libgdn.so only when nothing is built (tests load what is there)."""
    from gated_delta_rule_varlen_amd import build

    if not os.path.exists(build.LIB):
        build.build()


def dev(raw, dtype):
    """numpy storage (float32 or uint16 bits) -> device tensor of the named dtype."""
    import torch

    if raw is None:
        return None
    raw = np.ascontiguousarray(raw)
    if dtype == "f32":
        return torch.from_numpy(raw.astype(np.float32, copy=False)).cuda()
    t = torch.from_numpy(raw.view(np.int16)).cuda()
    return t.view(getattr(torch, TORCH_DT[dtype]))


def dev_i32(a):
    import torch

    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


def f64(t) -> np.ndarray:
    """Device tensor -> float64 numpy (exact for every dtype here)."""
    return t.float().cpu().numpy().astype(np.float64)


def bits(t) -> np.ndarray:
    """Raw bit patterns of a device tensor, for bit-exact comparisons."""
    import torch

    t = t.contiguous()
    if t.element_size() == 4:
        return t.view(torch.int32).cpu().numpy()
    return t.view(torch.int16).cpu().numpy()


def max_rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    """Normwise error: max |got - ref| / max |ref| over the compared elements."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    if ref.size == 0:
        return 0.0
    den = np.max(np.abs(ref))
    num = np.max(np.abs(got - ref))
    if not np.isfinite(num):
        return float("inf")
    return float(num / den) if den > 0 else float(num)


def elementwise_err(got: np.ndarray, ref: np.ndarray) -> float:
    """Diagnostic: max |got - ref| / (|ref| + 1e-3 max |ref|), elementwise."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    if ref.size == 0:
        return 0.0
    d = np.abs(got - ref)
    if not np.all(np.isfinite(d)):
        return float("inf")
    return float(np.max(d / (np.abs(ref) + 1e-3 * np.max(np.abs(ref)) + 1e-300)))


def assert_close(got, ref, tol, what):
    err = max_rel_err(got, ref)
    eerr = elementwise_err(got, ref)
    RECORD.append((os.environ.get("PYTEST_CURRENT_TEST", "").split(" ")[0], what, err, eerr, tol))
    print(f"[err] {what}: normwise {err:.3e} elementwise {eerr:.3e} (gate {tol:.1e})", flush=True)
    assert err <= tol, f"{what}: max relative error {err:.3e} > {tol:.1e}"
    return err


def assert_close_slices(got, ref, lengths, tol, what, *, token_major=True):
    """The normwise error of each (sequence, head) slice against that slice's own max |ref|, so an
    error confined to one short or small sequence or head cannot hide under another's magnitude.
    Token-major arrays are [N, H, ...] split by the sequence lengths; otherwise [B, H, ...]."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    worst = 0.0
    if token_major:
        start = 0
        for b, n in enumerate(lengths):
            for h in range(ref.shape[1]):
                r = ref[start:start + n, h]
                if r.size and np.max(np.abs(r)) > 0:
                    e = max_rel_err(got[start:start + n, h], r)
                    worst = max(worst, e)
                    assert e <= tol, f"{what}: sequence {b} head {h}: max relative error {e:.3e} > {tol:.1e}"
            start += n
    else:
        for b in range(ref.shape[0]):
            for h in range(ref.shape[1]):
                r = ref[b, h]
                if np.max(np.abs(r)) > 0:
                    e = max_rel_err(got[b, h], r)
                    worst = max(worst, e)
                    assert e <= tol, f"{what}: sequence {b} head {h}: max relative error {e:.3e} > {tol:.1e}"
    RECORD.append((os.environ.get("PYTEST_CURRENT_TEST", "").split(" ")[0], what + " per slice", worst, worst, tol))
    return worst


def sentinel(shape, dtype, device="cuda"):
    """A tensor filled with a NaN bit pattern (0x7fc0 / 0x7fc00000 family)."""
    import torch

    t = torch.empty(shape, dtype=getattr(torch, TORCH_DT[dtype]) if isinstance(dtype, str) else dtype, device=device)
    if t.element_size() == 4:
        t.view(torch.int32).fill_(0x7FC0DEAD)
    else:
        t.view(torch.int16).fill_(0x7E5A)
    return t


def head_subproblem(w: workloads.Workload, h: int, vsel=None):
    """One value head h (and its key head) of a workload, optionally restricted to the value
    columns vsel: inputs for an oracle run with HQ = H = 1."""
    G = w.H // w.HQ
    kh = h // G
    K, V = w.K, w.V
    vsel = np.arange(V) if vsel is None else np.asarray(vsel)
    q = w.qkv[:, kh * K:(kh + 1) * K]
    k = w.qkv[:, w.HQ * K + kh * K:w.HQ * K + (kh + 1) * K]
    v = w.qkv[:, 2 * w.HQ * K + h * V:2 * w.HQ * K + (h + 1) * V][:, vsel]
    qkv = np.ascontiguousarray(np.concatenate([q, k, v], axis=1))
    sub = dict(qkv=qkv, HQ=1, H=1, K=K, V=len(vsel), qkv_dtype=w.io, gate_dtype=w.gate_dtype,
               a=None if w.a is None else np.ascontiguousarray(w.a[:, h:h + 1]),
               b=None if w.b is None else np.ascontiguousarray(w.b[:, h:h + 1]),
               A_log=None if w.A_log is None else w.A_log[h:h + 1].copy(),
               dt_bias=None if w.dt_bias is None else w.dt_bias[h:h + 1].copy(),
               state_in=None if w.state is None else np.ascontiguousarray(w.state[:, h:h + 1][:, :, vsel]),
               l2norm=w.l2norm, softplus=w.softplus, sigmoid=w.sigmoid, scale=w.scale)
    return sub, vsel


def channel_subproblem(w: workloads.Workload, chans):
    """The conv restricted to the channels chans (the conv is depthwise)."""
    chans = np.asarray(chans)
    return dict(x=np.ascontiguousarray(w.x[:, chans]), w=np.ascontiguousarray(w.conv_w[chans]),
                bias=None if w.conv_bias is None else np.ascontiguousarray(w.conv_bias[chans]),
                state_in=None if w.conv_state is None else np.ascontiguousarray(w.conv_state[:, chans]),
                W=w.W, D=w.D, x_dtype=w.io, state_dtype=w.conv_state_dtype, silu=w.silu)
