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


def assert_close(got, ref, tol, what):
    err = max_rel_err(got, ref)
    assert err <= tol, f"{what}: max relative error {err:.3e} > {tol:.1e}"
    return err


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
